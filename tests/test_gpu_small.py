"""GPU parity on shapes the oracle finishes in seconds: the HIP path through
the C ABI against the CPU oracle, element by element on the fp32 logits,
plus the scheduling invariants of the "model-as-a-kernel" page (chunked ==
token by token, batched == alone, repeated runs identical), on the GPU."""
import dataclasses

import numpy as np
import pytest

from tests.parity import logits_ok, tokens_ok
from transformer_forward_pass_amd import synth

pytestmark = pytest.mark.gpu

TINY = synth.SHAPES["tiny"]

# ragged shapes: K with few lanes per row (K=344 -> 43 chunks), vocab not a
# multiple of any tile, head_dim 32/128, MQA, 8 query heads per kv head,
# qk-norm, tied and untied, zero layers
RAGGED = {
    "k344-v1000": synth.small_shape(n_layers=2, hidden=192, n_q_heads=6, n_kv_heads=2, head_dim=32,
                                    intermediate=344, vocab=1000),
    "qknorm-d128-mqa-tied": synth.small_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=1,
                                              head_dim=128, intermediate=512, vocab=777,
                                              qk_norm=True, tie_embeddings=True),
    "rep8": synth.small_shape(n_layers=3, hidden=512, n_q_heads=8, n_kv_heads=1, head_dim=64,
                              intermediate=1376, vocab=2051),
    "zero-layers": synth.small_shape(n_layers=0, vocab=3000),
}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    return torch


def _model(shape, max_seq=64, max_batch=None, seed=0):
    from transformer_forward_pass_amd import mak
    w = synth.make_weights(shape, seed)
    return w, mak.MakModel(shape, w, max_seq=max_seq, max_batch=max_batch)


def _np(t):
    return t.double().cpu().numpy()


def _ids(shape, n, seed=1):
    return [int(t) for t in np.random.default_rng(seed).integers(0, shape.vocab, n)]


def test_tiny_workload_generate_and_teacher_forced_logits(torch_cuda, orc):
    wl = synth.WORKLOADS["tiny"]
    w, m = _model(TINY)
    prompt = synth.make_prompts(wl)[0]
    got = m.generate(prompt, wl.max_new)
    ref, gaps, lgs = orc.Oracle(TINY, w, max_len=64).generate(prompt, wl.max_new, keep_logits=True)
    tokens_ok(got, ref, gaps, "tiny")
    lg = _np(m.prefill(prompt))
    exact = []
    for t in range(wl.max_new):
        exact.append(logits_ok(lg, lgs[t], "tiny step %d" % t)[2])
        if t + 1 < wl.max_new:
            lg = _np(m.decode_step(ref[t], len(prompt) + t)[0])
    print("tiny: bitwise-equal logit fraction min %.4f mean %.4f" % (min(exact), np.mean(exact)))


@pytest.mark.parametrize("chunk", [8, 16])
@pytest.mark.parametrize("name", sorted(RAGGED))
def test_ragged_shapes_teacher_forced(torch_cuda, orc, name, chunk):
    s = RAGGED[name]
    w, m = _model(s)
    m.set_prefill_chunk(chunk)
    ids = _ids(s, 13)                                  # chunks of 8 + 5, or one of 13
    o = orc.Oracle(s, w, max_len=64)
    logits_ok(_np(m.prefill(ids)), o.prefill(ids), name + " prefill")
    tok = 7
    for i in range(6):
        pos = len(ids) + i
        a, _ = m.decode_step(tok, pos)
        logits_ok(_np(a), o.decode_step(tok, pos), "%s step %d" % (name, i))
        tok = (tok * 31 + 5) % s.vocab


def test_next_token_is_lowest_index_argmax(torch_cuda):
    s = RAGGED["k344-v1000"]
    _, m = _model(s)
    for pos, tok in enumerate(_ids(s, 10)):
        lg, nxt = m.decode_step(tok, pos)
        v = _np(lg)
        assert nxt == int(np.flatnonzero(v == v.max())[0])


def test_kv_cache_matches_oracle_bitwise(torch_cuda, orc):
    """K (after rope) and V of every layer along a 20-token sequence."""
    s = RAGGED["qknorm-d128-mqa-tied"]
    w, m = _model(s)
    ids = _ids(s, 20)
    m.prefill(ids, want_logits=False)
    o = orc.Oracle(s, w, max_len=64)
    o.prefill(ids)
    for l in range(s.n_layers):
        k, v = m.read_kv(l, 0, 0, len(ids))
        assert np.array_equal(k, o.K[0][l][:, :len(ids)]), "layer %d K" % l
        assert np.array_equal(v, o.V[0][l][:, :len(ids)]), "layer %d V" % l


def test_chunked_prefill_equals_token_by_token_on_gpu(torch_cuda):
    s = RAGGED["k344-v1000"]
    _, m = _model(s)
    ids = _ids(s, 19)
    a = _np(m.prefill(ids))
    for i, t in enumerate(ids[:-1]):
        m.decode_step(t, i, want_logits=False)
    b = _np(m.decode_step(ids[-1], len(ids) - 1)[0])
    assert np.array_equal(a, b)


def test_batch_equals_alone_on_gpu_and_matches_oracle(torch_cuda, orc):
    s = dataclasses.replace(TINY, max_batch=4)
    w, m = _model(s, max_batch=4)
    prompts = [_ids(s, n, seed=10 + n) for n in (5, 12, 9)]
    for b, p in enumerate(prompts):
        m.prefill(p, slot=b, want_logits=False)
    toks = [3, 1000, 4095]
    pos = [len(p) for p in prompts]
    out, lg = m.decode_batch(toks, pos, slots=[0, 1, 2], steps=4)
    lg = _np(lg)
    for b, p in enumerate(prompts):
        w2, m2 = _model(s, max_batch=4)
        m2.prefill(p, slot=b, want_logits=False)
        out2, lg2 = m2.decode_batch([toks[b]], [pos[b]], slots=[b], steps=4)
        assert np.array_equal(out[:, b], out2[:, 0])
        assert np.array_equal(lg[b], _np(lg2)[0])
        o = orc.Oracle(s, w, max_len=64)
        o.prefill(p)
        t = toks[b]
        for st in range(4):
            ref = o.decode_step(t, pos[b] + st)
            if st == 3:
                logits_ok(lg[b], ref, "batch col %d" % b)
            t = int(np.argmax(ref))
            if t != out[st, b]:
                break


def test_repeated_generation_is_bitwise_identical(torch_cuda):
    _, m = _model(TINY)
    p = _ids(TINY, 16)
    runs = [m.generate(p, 24) for _ in range(3)]
    assert runs[0] == runs[1] == runs[2]
    a = _np(m.prefill(p))
    b = _np(m.prefill(p))
    assert np.array_equal(a, b)


def test_rewind_and_error_paths_leave_state_unchanged(torch_cuda):
    from transformer_forward_pass_amd import mak
    _, m = _model(TINY, max_seq=32)
    p = _ids(TINY, 10)
    base = _np(m.prefill(p))
    assert m.slot_length(0) == 10
    with pytest.raises(mak.MakError) as e:
        m.decode_step(1, 11)                          # beyond cached length
    assert e.value.code == mak.MAK_ERANGE
    with pytest.raises(mak.MakError):
        m.decode_step(TINY.vocab, 10)                 # token out of range
    with pytest.raises(mak.MakError):
        m.generate(p, 40)                             # exceeds max_seq
    assert m.slot_length(0) == 10
    # rewinding to position 9 and re-feeding the last prompt token reproduces the logits
    again = _np(m.decode_step(p[-1], 9)[0])
    assert np.array_equal(again, base)


def test_graph_replays_equal_phase_per_launch_bitwise(torch_cuda):
    """The captured-graph executor equals the phase-per-launch executor
    bitwise ("model-as-a-kernel", Method: the phase-per-launch debug mode is
    bitwise identical to the fused mode), on every one of several replays
    with unrelated eager GPU work and synchronisations in between."""
    from transformer_forward_pass_amd import mak
    s = dataclasses.replace(TINY, max_batch=2)
    _, m = _model(s, max_batch=2)
    p = _ids(s, 13)
    m.set_executor(mak.EXEC_PHASED)
    ref_tok = m.generate(p, 12)
    ref_pre = _np(m.prefill(p))
    m.prefill(p[:7], slot=1, want_logits=False)
    ref_bt, ref_bl = m.decode_batch([5, 6], [13, 7], slots=[0, 1], steps=3)
    ref_bl = _np(ref_bl)
    m.set_executor(mak.EXEC_GRAPH)
    junk = torch_cuda.randn(1 << 20, device="cuda")
    for rep in range(3):
        assert m.generate(p, 12) == ref_tok, "replay %d" % rep
        junk = (junk * 1.0001).sin()                 # unrelated eager work
        torch_cuda.cuda.synchronize()
        assert np.array_equal(_np(m.prefill(p)), ref_pre), "replay %d" % rep
        m.prefill(p[:7], slot=1, want_logits=False)
        bt, bl = m.decode_batch([5, 6], [13, 7], slots=[0, 1], steps=3)
        assert np.array_equal(bt, ref_bt) and np.array_equal(_np(bl), ref_bl), "replay %d" % rep
