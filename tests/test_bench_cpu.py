"""bench.py on the CPU: the one-GPU contract (--gpus N > 1 exits with a
message), the algorithmic byte accounting it reports rooflines with, and the
traffic lookup.  No GPU work."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from transformer_forward_pass_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_workloads_named_by_bench_exist():
    for name in (bench.WORKLOAD, bench.SECONDARY, "tinyllama-1.1b", "tinyllama-1.1b-b16", "qwen3-0.6b"):
        assert name in synth.WORKLOADS


@pytest.mark.parametrize("name", sorted(synth.SHAPES))
def test_gemv_bytes_are_the_weights_plus_vectors(name):
    s = synth.SHAPES[name]
    H, I, V = s.hidden, s.intermediate, s.vocab
    per_layer = sum(bench._gemv_bytes(s, k) for k in ("qkv", "o", "gateup", "down"))
    weights = 2 * ((s.q_dim + 2 * s.kv_dim) * H + H * s.q_dim + 2 * I * H + H * I)
    assert weights < per_layer < weights + 64 * (H + I + s.q_dim + s.kv_dim)
    assert 2 * V * H < bench._gemv_bytes(s, "lmhead") < 2 * V * H + 8 * V + 8 * H


def test_attention_bytes_count_each_cached_position_once():
    s = synth.SHAPES["smollm2-135m"]
    total, launches = bench._attn_bytes(s, 32, 128)
    assert launches == (4 + 127) * s.n_layers
    row = 2 * s.head_dim
    kv_reads = 0
    for t0 in range(0, 32, 8):
        kv_reads += 2 * s.n_kv_heads * (t0 + 8) * row
    for i in range(127):
        kv_reads += 2 * s.n_kv_heads * (32 + i + 1) * row
    assert total > kv_reads * s.n_layers
    assert total < 1.2 * kv_reads * s.n_layers


def test_traffic_lookup_is_none_or_a_byte_count():
    for kind in ("qkv", "attn", "o", "gateup", "down", "lmhead"):
        t = bench.measured_traffic(kind)
        assert t is None or (isinstance(t, int) and t > 0)
