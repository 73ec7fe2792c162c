"""mak_decode_step_static, the decode step that allocates nothing (its step
scratch lives in a static device array), against mak_decode_step through
the C ABI: logits, next token and the KV rows the step writes must be
bitwise equal, on two calls in a row where the second runs a smaller model
at a shorter context (the static array then still holds the first call's
larger contents).  A shape that needs more step scratch than the array
holds is rejected with MAK_EINVAL before any device work."""
import numpy as np
import pytest

from transformer_forward_pass_amd import synth

pytestmark = pytest.mark.gpu

BIG = synth.small_shape(n_layers=2, hidden=256, n_q_heads=8, n_kv_heads=2, head_dim=64,
                        intermediate=688, vocab=5000)
SMALL = synth.small_shape(n_layers=2, hidden=128, n_q_heads=4, n_kv_heads=1, head_dim=32,
                          intermediate=344, vocab=1000)
# the same step with 4-bit (MXFP4) per-layer weights
SMALL4 = synth.small_shape(n_layers=2, hidden=128, n_q_heads=4, n_kv_heads=1, head_dim=32,
                           intermediate=352, vocab=1000, weight_format="mxfp4")


def _ids(shape, n, seed):
    return [int(t) for t in np.random.default_rng(seed).integers(0, shape.vocab, n)]


def _pair(shape, max_seq):
    from transformer_forward_pass_amd import mak
    w = synth.make_weights(shape)
    return mak.MakModel(shape, w, max_seq=max_seq), mak.MakModel(shape, w, max_seq=max_seq)


def test_static_step_equals_decode_step_on_two_calls_in_a_row():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    # first call: 300 cached positions with split-KV attention (scores,
    # chunk maxima and partial outputs in the static array); second: a
    # smaller model at 9 positions through the single-pass attention; third:
    # a 4-bit model of that size
    for shape, ctx, split, seed in ((BIG, 300, True, 5), (SMALL, 9, False, 6), (SMALL4, 9, False, 7)):
        a, b = _pair(shape, 512)
        prompt = _ids(shape, ctx, seed)
        la = a.prefill(prompt)
        lb = b.prefill(prompt)
        assert torch.equal(la, lb)
        if split:
            a.set_attention_split(0)
            b.set_attention_split(0)
        tok, pos = int(torch.argmax(la).item()), ctx
        d_lg = torch.full((shape.vocab,), float("nan"), dtype=torch.float32, device="cuda")
        d_nx = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        ref_lg, ref_nx = a.decode_step(tok, pos)
        b.decode_step_static(tok, pos, d_lg, d_nx)
        torch.cuda.synchronize()
        assert torch.equal(d_lg, ref_lg), (shape.vocab, ctx)
        assert int(d_nx.item()) == ref_nx
        for layer in range(shape.n_layers):
            ka, va = a.read_kv(layer, 0, 0, pos + 1)
            kb, vb = b.read_kv(layer, 0, 0, pos + 1)
            assert np.array_equal(ka, kb) and np.array_equal(va, vb)
        assert b.slot_length(0) == pos + 1
        a.free()
        b.free()


def test_static_step_rejects_a_shape_beyond_the_static_scratch():
    import torch
    from transformer_forward_pass_amd import mak
    assert torch.cuda.is_available(), "GPU test without a GPU"
    shape = synth.small_shape(n_layers=1, hidden=256, n_q_heads=32, n_kv_heads=1, head_dim=16,
                              intermediate=256, vocab=512)
    m = mak.MakModel(shape, synth.make_weights(shape), max_seq=40000)
    m.prefill([1, 2, 3], want_logits=False)
    d_lg = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    with pytest.raises(mak.MakError) as e:
        m.decode_step_static(4, 3, d_lg, None)
    assert e.value.code == mak.MAK_EINVAL and "static scratch" in str(e.value)
    assert m.slot_length(0) == 3
    assert not torch.any(d_lg != 0)
    m.free()
