"""GPU parity of 4-bit (OCP MXFP4) weights: the library quantizes the
per-layer linear matrices at load and decodes from the 4-bit stream
("model-as-a-kernel", API section, "Supported" paragraph: 4-bit weights).
The oracle runs the same model on the dequantized weights (every dequantized
value is exactly bf16, oracle/mxfp4.py).  Shapes cover one to 64 lanes per
row, several batches per tile (K = 704 and 4160), ragged row tiles, GQA, MQA
with qk-norm at head_dim 128 and 16, and the 1B shape's K = 2048 layout."""
import dataclasses

import numpy as np
import pytest

from tests.parity import logits_ok
from transformer_forward_pass_amd import synth

pytestmark = pytest.mark.gpu

Q4 = {
    # hidden 256 (8 lanes per row), down K = 704 (2 lanes per row, 11 blocks per lane: two batches)
    "tiny4": synth.small_shape(intermediate=704, weight_format="mxfp4"),
    # 3 blocks per row: one lane per row, 64-row tiles, O/gate-up/down tiles ragged
    "ragged4-d16": synth.small_shape(n_layers=2, hidden=96, n_q_heads=6, n_kv_heads=1, head_dim=16,
                                     intermediate=160, vocab=777, weight_format="mxfp4"),
    "qknorm4-d128-mqa": synth.small_shape(n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=1, head_dim=128,
                                          qk_norm=True, tie_embeddings=True, intermediate=1024, vocab=1000,
                                          weight_format="mxfp4"),
    # down K = 4160: 65 blocks per lane, nine batches per tile
    "wide4": synth.small_shape(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                               intermediate=4160, vocab=2051, weight_format="mxfp4"),
    # the 1B layer layout: K = 2048, 64 lanes per row, one block per lane
    "l1-k2048": synth.small_shape(n_layers=1, hidden=2048, n_q_heads=32, n_kv_heads=8, head_dim=64,
                                  intermediate=2048, vocab=4096, weight_format="mxfp4"),
}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    return torch


def _model(shape, max_seq=64, max_batch=None, seed=0, w=None):
    from transformer_forward_pass_amd import mak
    w = synth.make_weights(shape, seed) if w is None else w
    return w, mak.MakModel(shape, w, max_seq=max_seq, max_batch=max_batch)


def _np(t):
    return t.double().cpu().numpy()


def _ids(shape, n, seed=1):
    return [int(t) for t in np.random.default_rng(seed).integers(0, shape.vocab, n)]


@pytest.mark.parametrize("chunk", [8, 16])
@pytest.mark.parametrize("name", sorted(Q4))
def test_mxfp4_shapes_teacher_forced(torch_cuda, orc, name, chunk):
    s = Q4[name]
    print("case", name, "chunk", chunk, flush=True)
    w, m = _model(s)
    m.set_prefill_chunk(chunk)
    ids = _ids(s, 13)                                   # chunks of 8 + 5, or one of 13
    o = orc.Oracle(s, w, max_len=64)
    exact = [logits_ok(_np(m.prefill(ids)), o.prefill(ids), name + " prefill")[2]]
    tok = 7
    for i in range(6):
        pos = len(ids) + i
        a, nxt = m.decode_step(tok, pos)
        ref = o.decode_step(tok, pos)
        exact.append(logits_ok(_np(a), ref, "%s step %d" % (name, i))[2])
        tok = nxt
    print("%s: bitwise-equal logit fraction min %.4f" % (name, min(exact)))


def test_mxfp4_equals_bf16_model_on_dequantized_weights(torch_cuda):
    """A 4-bit model and a bf16 model loaded with the oracle's dequantized
    weights give bitwise-identical logits: every dot product is exact before
    its single rounding on both paths."""
    from oracle import mxfp4
    s4 = Q4["tiny4"]
    s16 = dataclasses.replace(s4, weight_format="bf16")
    w, m4 = _model(s4)
    _, m16 = _model(s16, w=mxfp4.dequantized_weights(s16, w))
    ids = _ids(s4, 11)
    assert np.array_equal(_np(m4.prefill(ids)), _np(m16.prefill(ids)))
    tok = 3
    for i in range(5):
        a, n4 = m4.decode_step(tok, len(ids) + i)
        b, n16 = m16.decode_step(tok, len(ids) + i)
        assert np.array_equal(_np(a), _np(b)) and n4 == n16, "step %d" % i
        tok = n4


@pytest.mark.parametrize("chunk", [8, 16])
def test_mxfp4_chunked_prefill_equals_token_by_token(torch_cuda, chunk):
    s = Q4["wide4"]
    _, m = _model(s)
    m.set_prefill_chunk(chunk)
    ids = _ids(s, 21)
    a = _np(m.prefill(ids))
    for i, t in enumerate(ids[:-1]):
        m.decode_step(t, i, want_logits=False)
    b = _np(m.decode_step(ids[-1], len(ids) - 1)[0])
    assert np.array_equal(a, b)


def test_mxfp4_batch_equals_alone_and_matches_oracle(torch_cuda, orc):
    s = dataclasses.replace(Q4["qknorm4-d128-mqa"], max_batch=5)
    w, m = _model(s, max_batch=5)
    prompts = [_ids(s, n, seed=20 + n) for n in (5, 12, 9, 3, 7)]
    for b, p in enumerate(prompts):
        m.prefill(p, slot=b, want_logits=False)
    toks = [3, 999, 17, 500, 1]
    pos = [len(p) for p in prompts]
    out, lg = m.decode_batch(toks, pos, slots=list(range(5)), steps=3)
    lg = _np(lg)
    for b, p in enumerate(prompts):
        _, m2 = _model(s, max_batch=5, w=w)
        m2.prefill(p, slot=b, want_logits=False)
        out2, lg2 = m2.decode_batch([toks[b]], [pos[b]], slots=[b], steps=3)
        assert np.array_equal(out[:, b], out2[:, 0])
        assert np.array_equal(lg[b], _np(lg2)[0])
        o = orc.Oracle(s, w, max_len=64)
        o.prefill(p)
        t = toks[b]
        for st in range(3):
            ref = o.decode_step(t, pos[b] + st)
            if st == 2:
                logits_ok(lg[b], ref, "batch col %d" % b)
            t = int(np.argmax(ref))
            if t != out[st, b]:
                break


def test_mxfp4_kv_cache_matches_oracle_bitwise(torch_cuda, orc):
    s = Q4["ragged4-d16"]
    w, m = _model(s)
    ids = _ids(s, 20)
    m.prefill(ids, want_logits=False)
    o = orc.Oracle(s, w, max_len=64)
    o.prefill(ids)
    for l in range(s.n_layers):
        k, v = m.read_kv(l, 0, 0, len(ids))
        assert np.array_equal(k, o.K[0][l][:, :len(ids)]), "layer %d K" % l
        assert np.array_equal(v, o.V[0][l][:, :len(ids)]), "layer %d V" % l


def test_mxfp4_graph_equals_phased(torch_cuda):
    from transformer_forward_pass_amd import mak
    s = Q4["tiny4"]
    _, m = _model(s)
    p = _ids(s, 13)
    m.set_executor(mak.EXEC_PHASED)
    ref = m.generate(p, 10)
    m.set_executor(mak.EXEC_GRAPH)
    for rep in range(2):
        assert m.generate(p, 10) == ref, "replay %d" % rep
