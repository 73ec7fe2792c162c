"""Steps of 2..8 columns on the fp64 matrix cores (v_mfma_f64_4x4x4_4b_f64,
k_gemm8), which the planner picks for GEMMs of at least 2048 inputs and
2048 rows, with tiles of 8 rows for raw inputs whose 16-row groups would be
fewer than the CUs.  Three one-layer shapes inside that region run every
epilogue through it: QKV (RMSNorm inputs, store), O (raw inputs, residual),
gate/up (RMSNorm inputs, SwiGLU), down (raw inputs, residual) and the LM
head (RMSNorm inputs, logits and greedy argmax); O and down on 8-row tiles,
the rest on 16-row tiles (the second shape: a 3072-row gate/up and a
6144-row LM head; its 1536-input down stays on the vector units).  With 11
and 16 sequences O and down run as four groups of four columns on
half-height tiles, the rest on the 16x16 instruction (k_gemm16).  The third
shape takes workgroups of 2 and 4 row tiles (its gate/up and LM head) and a
down projection of 8192 inputs on half-height tiles.  Batched
decode must equal decoding each sequence alone (the one-column kernels)
bitwise, a chunked prompt must equal token-by-token consumption bitwise, and
both must match the CPU oracle ("model-as-a-kernel", API: decode_batch and chunked
prompt consumption; every dot product exact before its single rounding)."""
import numpy as np
import pytest

from tests.parity import logits_ok
from transformer_forward_pass_amd import synth

pytestmark = pytest.mark.gpu

SHAPES = {
    "i2048": synth.small_shape(n_layers=1, hidden=2048, n_q_heads=16, n_kv_heads=4, head_dim=128,
                               intermediate=2048, vocab=2048, max_batch=16),
    "i1536": synth.small_shape(n_layers=1, hidden=2048, n_q_heads=16, n_kv_heads=4, head_dim=128,
                               intermediate=1536, vocab=6144, max_batch=16),
    # workgroups of 2 row tiles (a 16384-row gate/up) and 4 (a 33000-row LM
    # head), and a down projection of 8192 inputs on half-height tiles
    "i8192": synth.small_shape(n_layers=1, hidden=2048, n_q_heads=16, n_kv_heads=4, head_dim=128,
                               intermediate=8192, vocab=33000, max_batch=16),
}
STEPS = 3


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    return torch


_W = {}


def _weights(name):
    if name not in _W:
        _W[name] = synth.make_weights(SHAPES[name])
    return _W[name]


def _np(t):
    return t.double().cpu().numpy()


def _prompts(shape, n, seed=5):
    rng = np.random.default_rng(seed)
    lens = rng.integers(3, 17, n)
    return [[int(t) for t in rng.integers(0, shape.vocab, int(k))] for k in lens]


@pytest.mark.parametrize("B", [16, 11, 8, 5, 2])
@pytest.mark.parametrize("name", sorted(SHAPES))
def test_batch_equals_alone_and_oracle(torch_cuda, orc, name, B):
    """B sequences decoded together (full and partial column groups) equal
    each decoded alone, tokens and logits, and match the oracle."""
    from transformer_forward_pass_amd import mak
    print("case %s B=%d" % (name, B), flush=True)
    SHAPE, weights = SHAPES[name], _weights(name)
    prompts = _prompts(SHAPE, B)
    bat = mak.MakModel(SHAPE, weights, max_seq=64, max_batch=16)
    one = mak.MakModel(SHAPE, weights, max_seq=64, max_batch=16)
    for b, p in enumerate(prompts):
        bat.prefill(p, slot=b, want_logits=False)
        one.prefill(p, slot=b, want_logits=False)
    toks = [(53 * b + 7) % SHAPE.vocab for b in range(B)]
    pos = [len(p) for p in prompts]
    out, lg = bat.decode_batch(toks, pos, slots=list(range(B)), steps=STEPS)
    lg = _np(lg)
    for b in range(B):
        o1, l1 = one.decode_batch([toks[b]], [pos[b]], slots=[b], steps=STEPS)
        assert np.array_equal(out[:, b], o1[:, 0]), "B=%d column %d tokens" % (B, b)
        assert np.array_equal(lg[b], _np(l1)[0]), "B=%d column %d logits" % (B, b)
    o = orc.Oracle(SHAPE, weights, max_len=64)
    o.prefill(prompts[B - 1])
    t = toks[B - 1]
    for st in range(STEPS):
        ref = o.decode_step(t, pos[B - 1] + st)
        t = int(out[st, B - 1])
    logits_ok(lg[B - 1], ref, "B=%d last column" % B)
    bat.free()
    one.free()


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_chunked_prompt_equals_token_by_token_and_oracle(torch_cuda, orc, name):
    """A 13-token prompt in chunks of 8 (steps of 8 and 5 columns) equals
    consuming it one token at a time, logits and KV cache bitwise, and
    matches the oracle."""
    from transformer_forward_pass_amd import mak
    print("case %s chunked" % name, flush=True)
    SHAPE, weights = SHAPES[name], _weights(name)
    ids = _prompts(SHAPE, 1, seed=9)[0] + _prompts(SHAPE, 1, seed=10)[0]
    ids = (ids * 2)[:13]
    runs = []
    for chunk in (8, 1):
        m = mak.MakModel(SHAPE, weights, max_seq=64)
        m.set_prefill_chunk(chunk)
        runs.append((m, _np(m.prefill(ids))))
    assert np.array_equal(runs[0][1], runs[1][1]), "chunk 8 != token by token"
    k8, v8 = runs[0][0].read_kv(0, 0, 0, len(ids))
    k1, v1 = runs[1][0].read_kv(0, 0, 0, len(ids))
    assert np.array_equal(k8, k1) and np.array_equal(v8, v1)
    logits_ok(runs[0][1], orc.Oracle(SHAPE, weights, max_len=64).prefill(ids), "chunked prompt")
    for m, _ in runs:
        m.free()
