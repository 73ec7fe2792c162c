"""Per-phase timing ("model-as-a-kernel", API section: decode_step_timed runs
the phases one launch each and reports per-phase milliseconds).

With timing on, every phase is its own launch carrying a pair of HIP events
stamped at the kernel's start and end.  The results must be bitwise the
same as the captured-graph run, each decode step must issue exactly the
phase launches of the program (five per layer, the LM head, and the
control-block update; split-KV attention adds two launches per layer), and
every timed phase must have taken a positive time."""
import numpy as np
import pytest

from transformer_forward_pass_amd import synth

pytestmark = pytest.mark.gpu

SHAPE = synth.small_shape(n_layers=3, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                          intermediate=688, vocab=4096)


def _model(max_seq=64):
    import torch
    from transformer_forward_pass_amd import mak
    assert torch.cuda.is_available(), "GPU test without a GPU"
    w = synth.make_weights(SHAPE)
    return mak.MakModel(SHAPE, w, max_seq=max_seq)


def _ids(n, seed=1):
    return [int(t) for t in np.random.default_rng(seed).integers(0, SHAPE.vocab, n)]


def test_timed_generation_equals_graph_generation_bitwise():
    m = _model()
    prompt = _ids(13)
    ref = m.generate(prompt, 12)
    lg_ref = m.prefill(prompt).cpu().numpy()
    step_ref = [m.decode_step(t, len(prompt) + i)[0].cpu().numpy() for i, t in enumerate(ref[:4])]
    m.set_phase_timing(True)
    got = m.generate(prompt, 12)
    lg = m.prefill(prompt).cpu().numpy()
    step = [m.decode_step(t, len(prompt) + i)[0].cpu().numpy() for i, t in enumerate(ref[:4])]
    m.set_phase_timing(False)
    assert got == ref
    assert np.array_equal(lg, lg_ref)
    for a, b in zip(step, step_ref):
        assert np.array_equal(a, b)
    m.free()


@pytest.mark.parametrize("split", [False, True], ids=["single-pass", "split-kv"])
def test_launches_per_decode_step_and_positive_times(split):
    m = _model()
    if split:
        m.set_attention_split(0)
    prompt = _ids(9)
    first = int(np.argmax(m.prefill(prompt).cpu().numpy()))
    L = SHAPE.n_layers
    m.set_phase_timing(True)
    n_steps = 5
    tok = first
    for i in range(n_steps):
        _, tok = m.decode_step(tok, len(prompt) + i)
    t = m.phase_times()
    m.set_phase_timing(False)
    per_step = {k: n // n_steps for k, (_, n) in t.items()}
    assert all(n % n_steps == 0 for _, n in t.values()), t
    expect = {"qkv": L, "attn": (3 if split else 1) * L, "o": L, "gateup": L, "down": L,
              "lmhead": 1, "ctl": 1}
    assert per_step == expect, (per_step, expect)
    # 5 launches per layer + LM head (+ control update, + 2 per layer when split)
    assert sum(per_step.values()) - 1 == 5 * L + 1 + (2 * L if split else 0)
    for k, (ms, n) in t.items():
        assert ms > 0.0, "phase %s: %d launches, %.6f ms" % (k, n, ms)
    m.free()


@pytest.mark.parametrize("chunk,steps", [(8, 2), (16, 1), (None, 1)])
def test_prefill_chunk_launches(chunk, steps):
    """A 13-token prompt in chunks of 8 takes two steps (8 + 5 tokens); in
    chunks of 16, the default, one step of 13.  The LM head runs once, for
    the last token."""
    m = _model()
    if chunk:
        m.set_prefill_chunk(chunk)
    L = SHAPE.n_layers
    m.set_phase_timing(True)
    m.prefill(_ids(13))
    t = m.phase_times()
    m.set_phase_timing(False)
    n = {k: v[1] for k, v in t.items()}
    assert n == {"qkv": steps * L, "attn": steps * L, "o": steps * L, "gateup": steps * L,
                 "down": steps * L, "lmhead": 1, "ctl": steps}, n
    m.free()
