"""Split-KV attention on the GPU: scores and a maximum per chunk of 128
positions, the exact global softmax and P.V per chunk, then the chunk sums
("model-as-a-kernel", Method section: split-KV with a deterministic
combine).  The split path must give exactly the single-pass results, and
both must match the CPU oracle, across several chunks, every head size, MQA
and GQA, qk-norm, chunked prefill and batched decode."""
import dataclasses

import numpy as np
import pytest

from tests.parity import logits_ok, tokens_ok
from transformer_forward_pass_amd import synth

pytestmark = pytest.mark.gpu

TINY = synth.SHAPES["tiny"]
SHAPES = {
    "tiny-d64-gqa": TINY,
    "d32-gqa3": synth.small_shape(n_layers=2, hidden=192, n_q_heads=6, n_kv_heads=2, head_dim=32,
                                  intermediate=344, vocab=1000),
    "d128-qknorm-mqa": synth.small_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=1, head_dim=128,
                                         intermediate=512, vocab=777, qk_norm=True, tie_embeddings=True),
    "d16-gqa4": synth.small_shape(n_layers=2, hidden=128, n_q_heads=8, n_kv_heads=2, head_dim=16,
                                  intermediate=256, vocab=500),
}
SINGLE = 1 << 30   # threshold that never splits (up to the single-pass capacity)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    return torch


def _model(shape, w, split_above, max_seq=512, max_batch=None):
    from transformer_forward_pass_amd import mak
    m = mak.MakModel(shape, w, max_seq=max_seq, max_batch=max_batch)
    m.set_attention_split(split_above)
    m.set_prefill_chunk(8)     # per-column split-KV (16-token prompt steps run blockwise)
    return m


def _np(t):
    return t.double().cpu().numpy()


def _ids(shape, n, seed=1):
    return [int(t) for t in np.random.default_rng(seed).integers(0, shape.vocab, n)]


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_split_equals_single_pass_and_oracle(torch_cuda, orc, name):
    """A 300-token prompt (chunks 0-2, the last one ragged) prefilled in chunks
    of 8, then teacher-forced decode steps: split-KV == single pass bitwise,
    both within tolerance of the oracle; KV cache bitwise equal to the oracle's."""
    s = SHAPES[name]
    w = synth.make_weights(s)
    ids = _ids(s, 300)
    sp, one = _model(s, w, 0), _model(s, w, SINGLE)
    o = orc.Oracle(s, w, max_len=512)
    a, b = _np(sp.prefill(ids)), _np(one.prefill(ids))
    assert np.array_equal(a, b), name + " prefill: split != single pass"
    logits_ok(a, o.prefill(ids), name + " prefill")
    tok = 11
    for i in range(5):
        pos = len(ids) + i
        a, na = sp.decode_step(tok, pos)
        b, nb = one.decode_step(tok, pos)
        assert na == nb and np.array_equal(_np(a), _np(b)), "%s step %d: split != single pass" % (name, i)
        logits_ok(_np(a), o.decode_step(tok, pos), "%s step %d" % (name, i))
        tok = (tok * 31 + 5) % s.vocab
    n = len(ids) + 5
    for l in range(s.n_layers):
        k, v = sp.read_kv(l, 0, 0, n)
        assert np.array_equal(k, o.K[0][l][:, :n]), "%s layer %d K" % (name, l)
        assert np.array_equal(v, o.V[0][l][:, :n]), "%s layer %d V" % (name, l)


def test_generate_switches_to_split_mid_sequence(torch_cuda, orc):
    """Threshold 256: a 240-token prompt + 40 new tokens crosses it
    mid-generation; tokens equal the never-split run and the oracle."""
    w = synth.make_weights(TINY)
    prompt = _ids(TINY, 240, seed=3)
    m = _model(TINY, w, 256)
    got = m.generate(prompt, 40)
    one = _model(TINY, w, SINGLE)
    assert got == one.generate(prompt, 40)
    ref, gaps, _ = orc.Oracle(TINY, w, max_len=512).generate(prompt, 40)
    tokens_ok(got, ref, gaps, "tiny 240+40")


def test_batched_decode_split_equals_single_pass(torch_cuda, orc):
    """Three sequences at 140, 260 and 300 cached positions decoded together."""
    s = dataclasses.replace(TINY, max_batch=4)
    w = synth.make_weights(s)
    prompts = [_ids(s, n, seed=20 + n) for n in (140, 260, 300)]
    runs = []
    for above in (0, SINGLE):
        m = _model(s, w, above, max_batch=4)
        for b, p in enumerate(prompts):
            m.prefill(p, slot=b, want_logits=False)
        out, lg = m.decode_batch([3, 1000, 4095], [len(p) for p in prompts], slots=[0, 1, 2], steps=3)
        runs.append((out, _np(lg)))
    assert np.array_equal(runs[0][0], runs[1][0]) and np.array_equal(runs[0][1], runs[1][1])
    o = orc.Oracle(s, w, max_len=512)
    o.prefill(prompts[2])
    t = 4095
    for st in range(3):
        ref = o.decode_step(t, len(prompts[2]) + st)
        t = int(runs[0][0][st, 2])
    logits_ok(runs[0][1][2], ref, "batch column 2 after 3 steps")
