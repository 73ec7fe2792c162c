"""Whole-model pins for the oracle.

* fp64 mode against a NumPy full-sequence forward written in the matrix
  form with an explicit causal mask ("GPT-2 on the GPU", section "The Whole
  Model as One Kernel": masking future positions gives them exactly zero
  weight), rope as complex multiplication and GQA as repeated KV heads --
  a different route to the same numbers than the oracle's incremental
  per-row KV-cache form.
* closed forms: zero layers; zero O and down projections.
* the scheduling invariants the "model-as-a-kernel" page claims (sections
  Method and Measured): chunked prefill == token by token, batched ==
  alone, and cached decode == full recompute, all bitwise in the oracle.
"""
import dataclasses
import os
import subprocess
import sys

import numpy as np
import pytest

from transformer_forward_pass_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SMALL = synth.small_shape(n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                          intermediate=96, vocab=97)
SMALL_QK = dataclasses.replace(SMALL, qk_norm=True, tie_embeddings=True, n_kv_heads=1)


def _f(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def numpy_forward_fp64(s, w, ids):
    """Full-sequence fp64 forward; logits of every position [T, V]."""
    T, d = len(ids), s.head_dim
    rep = s.n_q_heads // s.n_kv_heads
    pos = np.arange(T)

    def rms(x, wt):
        return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + s.rms_eps) * _f(wt)

    def rope(u):                                        # u [T, heads, d]
        ang = pos[:, None] * s.rope_theta ** (-2.0 * np.arange(d // 2) / d)
        z = (u[..., :d // 2] + 1j * u[..., d // 2:]) * np.exp(1j * ang)[:, None, :]
        return np.concatenate([z.real, z.imag], axis=-1)

    X = _f(w["embed"])[np.asarray(ids)]
    mask = np.triu(np.full((T, T), -np.inf), k=1)
    for lw in w["layers"]:
        h = rms(X, lw["attn_norm"])
        Q = (h @ _f(lw["wq"]).T).reshape(T, s.n_q_heads, d)
        K = (h @ _f(lw["wk"]).T).reshape(T, s.n_kv_heads, d)
        V = (h @ _f(lw["wv"]).T).reshape(T, s.n_kv_heads, d)
        if s.qk_norm:
            Q, K = rms(Q, lw["q_norm"]), rms(K, lw["k_norm"])
        Q, K = rope(Q), rope(K)
        K, V = np.repeat(K, rep, axis=1), np.repeat(V, rep, axis=1)
        S = np.einsum("thd,shd->hts", Q, K) / np.sqrt(d) + mask
        P = np.exp(S - S.max(-1, keepdims=True))
        P /= P.sum(-1, keepdims=True)
        O = np.einsum("hts,shd->thd", P, V).reshape(T, -1)
        X = X + O @ _f(lw["wo"]).T
        h2 = rms(X, lw["mlp_norm"])
        G, U = h2 @ _f(lw["w_gate"]).T, h2 @ _f(lw["w_up"]).T
        X = X + (G / (1 + np.exp(-G)) * U) @ _f(lw["w_down"]).T
    lm = w["embed"] if s.tie_embeddings else w["lm_head"]
    return rms(X, w["final_norm"]) @ _f(lm).T


def _ids(s, n, seed=1):
    return [int(t) for t in np.random.default_rng(seed).integers(0, s.vocab, n)]


@pytest.mark.parametrize("shape", [SMALL, SMALL_QK], ids=["gqa", "qknorm-mqa-tied"])
def test_fp64_mode_matches_numpy_masked_forward(orc, shape):
    w = synth.make_weights(shape)
    ids = _ids(shape, 11)
    o = orc.Oracle(shape, w, rounding=False, max_len=16)
    got = np.stack(o.forward([(0, t, p) for p, t in enumerate(ids)]))
    ref = numpy_forward_fp64(shape, w, ids)
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_rounded_mode_close_to_fp64(orc):
    w = synth.make_weights(SMALL)
    ids = _ids(SMALL, 9)
    a = orc.Oracle(SMALL, w, max_len=16).prefill(ids)
    b = orc.Oracle(SMALL, w, rounding=False, max_len=16).prefill(ids)
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 5e-2


def test_zero_layers_closed_form(orc):
    s = dataclasses.replace(SMALL, n_layers=0)
    w = synth.make_weights(s)
    t = 42
    x = _f(w["embed"][t])
    hf = x / np.sqrt(np.mean(x * x) + s.rms_eps) * _f(w["final_norm"])
    ref = _f(w["lm_head"]) @ hf
    got = orc.Oracle(s, w, rounding=False, max_len=4).decode_step(t, 0)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_zero_output_projections_leave_residual_untouched(orc):
    """W_o = W_down = 0: every block adds exactly zero, so the logits equal
    the zero-layer model's bitwise (rounded mode)."""
    w = synth.make_weights(SMALL)
    for lw in w["layers"]:
        lw["wo"] = np.zeros_like(lw["wo"])
        lw["w_down"] = np.zeros_like(lw["w_down"])
    s0 = dataclasses.replace(SMALL, n_layers=0)
    w0 = dict(w, layers=[])
    ids = _ids(SMALL, 5)
    a = orc.Oracle(SMALL, w, max_len=8).prefill(ids)
    b = orc.Oracle(s0, w0, max_len=8).prefill(ids)
    assert np.array_equal(a, b)


def test_gqa_equals_mha_with_repeated_kv_heads(orc):
    """Query head h reads kv head h // (Hq/Hkv): an MHA model whose K/V
    weights repeat each kv head's rows for its group gives identical logits."""
    w = synth.make_weights(SMALL)
    s_mha = dataclasses.replace(SMALL, n_kv_heads=SMALL.n_q_heads)
    d, rep = SMALL.head_dim, SMALL.n_q_heads // SMALL.n_kv_heads
    w_mha = dict(w, layers=[])
    for lw in w["layers"]:
        m = dict(lw)
        for k in ("wk", "wv"):
            heads = lw[k].reshape(SMALL.n_kv_heads, d, -1)
            m[k] = np.repeat(heads, rep, axis=0).reshape(SMALL.n_q_heads * d, -1)
        w_mha["layers"].append(m)
    ids = _ids(SMALL, 7)
    a = orc.Oracle(SMALL, w, max_len=8).prefill(ids)
    b = orc.Oracle(s_mha, w_mha, max_len=8).prefill(ids)
    assert np.array_equal(a, b)


def test_cached_decode_equals_full_recompute(orc):
    w = synth.make_weights(SMALL)
    ids = _ids(SMALL, 10)
    o = orc.Oracle(SMALL, w, max_len=16)
    step = [o.decode_step(t, p) for p, t in enumerate(ids)]
    full = orc.Oracle(SMALL, w, max_len=16).forward([(0, t, p) for p, t in enumerate(ids)])
    for a, b in zip(step, full):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("chunk", [3, 8])
def test_chunked_prefill_equals_token_by_token(orc, chunk):
    w = synth.make_weights(SMALL_QK)
    ids = _ids(SMALL_QK, 13)
    a = orc.Oracle(SMALL_QK, w, max_len=16).prefill(ids, chunk=chunk)
    b = orc.Oracle(SMALL_QK, w, max_len=16).prefill(ids, chunk=1)
    assert np.array_equal(a, b)


def test_batched_equals_alone(orc):
    w = synth.make_weights(SMALL)
    A, B = _ids(SMALL, 6, 2), _ids(SMALL, 4, 3)
    o = orc.Oracle(SMALL, w, max_len=16, n_seqs=2)
    o.prefill(A, seq=0)
    o.prefill(B, seq=1)
    both = o.forward([(0, 5, len(A)), (1, 9, len(B))])
    a1 = orc.Oracle(SMALL, w, max_len=16)
    a1.prefill(A)
    b1 = orc.Oracle(SMALL, w, max_len=16)
    b1.prefill(B)
    assert np.array_equal(both[0], a1.decode_step(5, len(A)))
    assert np.array_equal(both[1], b1.decode_step(9, len(B)))


def test_rewind_overwrites_cache(orc):
    """Decoding again at an earlier position replaces that position's K/V."""
    w = synth.make_weights(SMALL)
    o = orc.Oracle(SMALL, w, max_len=8)
    o.prefill([1, 2, 3])
    o.decode_step(50, 3)
    again = o.decode_step(60, 3)
    fresh = orc.Oracle(SMALL, w, max_len=8)
    fresh.prefill([1, 2, 3])
    assert np.array_equal(again, fresh.decode_step(60, 3))


def test_thread_count_independence(orc, tmp_path):
    code = (
        "import sys, numpy as np; sys.path.insert(0, %r)\n"
        "from oracle import oracle as O\n"
        "from transformer_forward_pass_amd import synth\n"
        "s = synth.small_shape(n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16,"
        " intermediate=96, vocab=97)\n"
        "w = synth.make_weights(s)\n"
        "np.save(sys.argv[1], O.Oracle(s, w, max_len=16).prefill(list(range(11))))\n" % ROOT)
    outs = []
    for n in ("1", "5"):
        f = tmp_path / ("l%s.npy" % n)
        env = dict(os.environ, OMP_NUM_THREADS=n)
        subprocess.run([sys.executable, "-c", code, str(f)], check=True, env=env)
        outs.append(np.load(f))
    assert np.array_equal(outs[0], outs[1])


def test_generate_contract(orc):
    """max_new tokens; the first comes from the prefill logits; each later
    token is the argmax of the step that consumed the previous one."""
    w = synth.make_weights(SMALL)
    p = _ids(SMALL, 5)
    toks, gaps, lgs = orc.Oracle(SMALL, w, max_len=16).generate(p, 4, keep_logits=True)
    assert len(toks) == 4 and len(gaps) == 4
    o = orc.Oracle(SMALL, w, max_len=16)
    lg = o.prefill(p)
    assert toks[0] == int(np.argmax(lg)) and np.array_equal(lg, lgs[0])
    for i in range(1, 4):
        lg = o.decode_step(toks[i - 1], len(p) + i - 1)
        assert toks[i] == int(np.argmax(lg))
