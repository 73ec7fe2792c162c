"""Blockwise split-KV attention for prompt chunks on the GPU.

A prefill step's columns are consecutive positions of one sequence, so its
split-KV attention runs one workgroup per (query head, 128-position chunk)
that serves every column of the step, with each column's causal limit, and
one softmax row per (column, head) ("CuTeDSL at Perplexity", section on
prefill and decode specialization; "model-as-a-kernel", Method section:
split-KV with a deterministic combine).  It must equal the per-column
split-KV kernels bitwise (logits and KV cache) for every head size, MQA and
GQA, qk-norm, chunk sizes that straddle the 128-position chunks, prompts
continued from a cached prefix, 4-bit weights and graph replays, and match
the CPU oracle."""
import numpy as np
import pytest

from tests.parity import logits_ok
from transformer_forward_pass_amd import synth

pytestmark = pytest.mark.gpu

SHAPES = {
    "tiny-d64-gqa": synth.SHAPES["tiny"],
    "d32-gqa3": synth.small_shape(n_layers=2, hidden=192, n_q_heads=6, n_kv_heads=2, head_dim=32,
                                  intermediate=344, vocab=1000),
    "d128-qknorm-mqa": synth.small_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=1, head_dim=128,
                                         intermediate=512, vocab=777, qk_norm=True, tie_embeddings=True),
    "d16-gqa4": synth.small_shape(n_layers=2, hidden=128, n_q_heads=8, n_kv_heads=2, head_dim=16,
                                  intermediate=256, vocab=500),
    "mxfp4-d64": synth.small_shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                                   intermediate=704, vocab=1000, weight_format="mxfp4"),
}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    return torch


def _model(shape, w, block, chunk, split_above=0, max_seq=512):
    from transformer_forward_pass_amd import mak
    m = mak.MakModel(shape, w, max_seq=max_seq)
    m.set_attention_split(split_above)
    m.set_block_attention(block)
    m.set_prefill_chunk(chunk)
    return m


def _np(t):
    return t.double().cpu().numpy()


def _ids(shape, n, seed=1):
    return [int(t) for t in np.random.default_rng(seed).integers(0, shape.vocab, n)]


def _same_kv(a, b, shape, n, what):
    for l in range(shape.n_layers):
        ka, va = a.read_kv(l, 0, 0, n)
        kb, vb = b.read_kv(l, 0, 0, n)
        assert np.array_equal(ka, kb) and np.array_equal(va, vb), "%s layer %d KV" % (what, l)


@pytest.mark.parametrize("chunk", [16, 5])
@pytest.mark.parametrize("name", sorted(SHAPES))
def test_block_equals_per_column_split_and_oracle(torch_cuda, orc, name, chunk):
    """A 300-token prompt with split-KV from the first chunk: chunks of 16
    (aligned to the 128-position chunks) and of 5 (steps 25 and 51 straddle
    positions 128 and 256).  Blockwise == per-column split bitwise, logits
    and KV cache; the logits match the oracle, the KV cache bitwise."""
    s = SHAPES[name]
    w = synth.make_weights(s)
    ids = _ids(s, 300)
    print("case", name, "chunk", chunk, flush=True)
    blk, col = _model(s, w, True, chunk), _model(s, w, False, chunk)
    a, b = _np(blk.prefill(ids)), _np(col.prefill(ids))
    assert np.array_equal(a, b), "%s chunk %d: blockwise != per-column split" % (name, chunk)
    _same_kv(blk, col, s, len(ids), name)
    if chunk == 16:
        o = orc.Oracle(s, w, max_len=512)
        logits_ok(a, o.prefill(ids), name + " blockwise prefill")
        for l in range(s.n_layers):
            k, v = blk.read_kv(l, 0, 0, len(ids))
            assert np.array_equal(k, o.K[0][l][:, :len(ids)]), "%s layer %d K" % (name, l)
            assert np.array_equal(v, o.V[0][l][:, :len(ids)]), "%s layer %d V" % (name, l)
    # decode continues from the blockwise cache exactly as from the other
    tok = 7
    for i in range(3):
        x, nx = blk.decode_step(tok, len(ids) + i)
        y, ny = col.decode_step(tok, len(ids) + i)
        assert nx == ny and np.array_equal(_np(x), _np(y)), "%s decode step %d" % (name, i)
        tok = nx
    blk.free()
    col.free()


def test_continued_prompt_and_threshold_crossing(torch_cuda, orc):
    """A cached 150-token prefix, then 170 more prompt tokens from position 150
    in chunks of 16 (the first step starts mid-chunk, at 150), with the split
    threshold at 200: steps below it run single-pass, the rest blockwise.
    Equal to the per-column split run and to one 320-token prefill, and the
    logits match the oracle."""
    s = SHAPES["d32-gqa3"]
    w = synth.make_weights(s)
    ids = _ids(s, 320, seed=4)
    runs = []
    for block in (True, False):
        m = _model(s, w, block, 16, split_above=200)
        m.prefill(ids[:150], want_logits=False)
        runs.append((m, _np(m.prefill(ids[150:], start_pos=150))))
    assert np.array_equal(runs[0][1], runs[1][1])
    _same_kv(runs[0][0], runs[1][0], s, 320, "continued")
    whole = _model(s, w, True, 16, split_above=200)
    assert np.array_equal(_np(whole.prefill(ids)), runs[0][1])
    logits_ok(runs[0][1], orc.Oracle(s, w, max_len=512).prefill(ids), "continued prompt")
    for m, _ in runs:
        m.free()
    whole.free()


def test_block_graph_replays_equal_phased(torch_cuda):
    """The captured prompt-chunk graph (blockwise attention) replayed for many
    steps and prompts equals the one-launch-per-phase run bitwise."""
    from transformer_forward_pass_amd import mak
    s = SHAPES["tiny-d64-gqa"]
    w = synth.make_weights(s)
    m = _model(s, w, True, 8)
    ref = []
    m.set_executor(mak.EXEC_PHASED)
    for seed in (1, 2):
        ref.append(_np(m.prefill(_ids(s, 200, seed=seed))))
    m.set_executor(mak.EXEC_GRAPH)
    for rep in range(2):
        for i, seed in enumerate((1, 2)):
            assert np.array_equal(_np(m.prefill(_ids(s, 200, seed=seed))), ref[i]), "replay %d seed %d" % (rep, seed)
    m.free()


def test_block_launches_per_prompt_step():
    """Prompt steps past the threshold launch four attention kernels per layer
    (scores, softmax, P.V, combine) blockwise and three per column-split;
    one-token steps never run blockwise."""
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    s = SHAPES["tiny-d64-gqa"]
    w = synth.make_weights(s)
    L = s.n_layers
    for block, per in ((True, 4), (False, 3)):
        m = _model(s, w, block, 8, max_seq=64)
        m.set_phase_timing(True)
        m.prefill(_ids(s, 17))                    # steps of 8, 8 and 1 tokens
        t = m.phase_times()
        m.set_phase_timing(False)
        n_attn = t["attn"][1]
        assert n_attn == (2 * per + 3) * L, (block, n_attn)
        m.free()
    from transformer_forward_pass_amd import mak
    m = _model(s, w, True, 8, max_seq=64)
    with pytest.raises(mak.MakError):
        m.set_block_attention(2)
    m.free()


@pytest.mark.parametrize("case", ["ragged-max-seq", "gqa8", "past-4096"])
def test_block_edges_equal_per_column_split(torch_cuda, case):
    """Edges of the (head, 128-position chunk) grid: a max_seq that is not a
    multiple of 128 (the last chunk ragged, the prompt ending in it), eight
    query heads per kv head (one KV-append owner among eight), and a prompt
    running past the 4096-position single-pass capacity.  Blockwise ==
    per-column split bitwise, logits and KV cache."""
    if case == "ragged-max-seq":
        s, n, max_seq, chunk = SHAPES["d32-gqa3"], 290, 300, 16
    elif case == "gqa8":
        s = synth.small_shape(n_layers=2, hidden=256, n_q_heads=8, n_kv_heads=1, head_dim=32,
                              intermediate=344, vocab=600)
        n, max_seq, chunk = 333, 512, 13
    else:
        s = synth.small_shape(n_layers=1, hidden=128, n_q_heads=2, n_kv_heads=1, head_dim=64,
                              intermediate=256, vocab=300)
        n, max_seq, chunk = 4200, 4224, 16
    w = synth.make_weights(s)
    ids = _ids(s, n, seed=9)
    print("case", case, flush=True)
    blk = _model(s, w, True, chunk, max_seq=max_seq)
    col = _model(s, w, False, chunk, max_seq=max_seq)
    a, b = _np(blk.prefill(ids)), _np(col.prefill(ids))
    assert np.array_equal(a, b), case
    _same_kv(blk, col, s, n, case)
    blk.free()
    col.free()
