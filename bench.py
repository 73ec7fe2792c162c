"""Greedy-decode benchmark on one MI355X.

One step = one mak_generate call of the SmolLM2-135M-shaped random-init model:
a 32-token prompt consumed in chunks of 16, then 128 greedy tokens at batch 1
with on-device token feedback -- every phase of the decode path (embedding
gather, RMSNorm, Q/K/V/O and SwiGLU GEMVs, rope, GQA attention over the KV
cache, LM head, argmax).  value = generated tokens per second over the K
timed steps (the "model-as-a-kernel" page's measurement: 128 greedy tokens
after a 32-token prompt, section "Measured").

Also printed, in the same JSON line:
  roofline      -- the dominant kernel (the phase kind with the largest total
                   GPU time: a GEMV kind or attention) measured with HIP events
                   on the model's stream over a second pass of the same K
                   steps: algorithmic bytes per launch / average launch
                   duration, against 8 TB/s.
  cpu_baseline  -- the CPU oracle on a bounded sample of the same workload.
  token_roofline -- bytes one decode token must stream (weights + KV) per
                   steady-state decode token time, against 8 TB/s.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_smollm2-135m.md")
TRAFFIC_SOURCES = ["gemv_kernels.h", "gemvn_kernels.h", "device_math.h", "mak_internal.h", "gemv1_swiglu.hip",
                   "gemv1_store.hip", "gemv1_residual.hip", "gemv1_logits.hip", "kernels.hip", "attn_split.hip"]


def measured_traffic(kind):
    """HBM bytes per launch of phase kind `kind` from the committed rocprofv3
    counter summary (FETCH_SIZE/WRITE_SIZE scaled by a copy of known size),
    or None when the summary is missing or the kernel sources changed since
    the counters were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        line = line.strip()
        if ":" in line and not line.startswith("|"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "transformer_forward_pass_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if vals.get("source_sha256") != h.hexdigest() or ("traffic." + kind) not in vals:
        return None
    return int(float(vals["traffic." + kind]))


WORKLOAD = "smollm2-135m"
SECONDARY = "llama-3.2-1b"


def _gemv_bytes(shape, kind):
    """Algorithmic bytes of one launch of a phase kind at batch 1: weight
    bytes streamed once + activation vectors read and written (bf16).  A
    4-bit (MXFP4) matrix of n weights streams n/2 code bytes and n/32 scale
    bytes; the LM head stays bf16."""
    H, I, d = shape.hidden, shape.intermediate, shape.head_dim
    qd, kvd = shape.q_dim, shape.kv_dim

    def wb(n):
        return n // 2 + n // 32 if getattr(shape, "weight_format", "bf16") == "mxfp4" else 2 * n
    if kind == "qkv":
        return wb((qd + 2 * kvd) * H) + 2 * (H + H) + 2 * (qd + 2 * kvd)
    if kind == "o":
        return wb(H * qd) + 2 * qd + 2 * 2 * H
    if kind == "gateup":
        return wb(2 * I * H) + 2 * (H + H) + 2 * I
    if kind == "down":
        return wb(H * I) + 2 * I + 2 * 2 * H
    if kind == "lmhead":
        return 2 * shape.vocab * H + 2 * (H + H) + 4 * shape.vocab
    return None


def _on_matrix_cores(shape, kind, ncols):
    """Whether the library's planner runs a multi-column GEMM of this kind on
    the fp64 matrix cores: 9-16 columns always (k_gemm16, or k_gemm8 as four
    column groups for raw inputs on few row groups); 2-8 columns where
    it picks k_gemm8 (at least 2048 inputs and 2048 rows, raw inputs -- O and
    down -- only at 2048 inputs)."""
    if ncols >= 9:
        return True
    if ncols < 2:
        return False
    H, I = shape.hidden, shape.intermediate
    n, k, staged = {"qkv": (shape.q_dim + 2 * shape.kv_dim, H, True), "o": (H, shape.q_dim, False),
                    "gateup": (2 * I, H, True), "down": (H, I, False), "lmhead": (shape.vocab, H, True)}[kind]
    return k >= 2048 and n >= 2048 and (staged or k == 2048)


def _attn_bytes(shape, p0, n_new, chunk=8):
    """Algorithmic bytes of the attention launches of one generate call
    (prompt of p0 tokens in chunks, then n_new - 1 decode steps), and their
    number of launches: per step, the K and V rows of every kv head at the
    positions attended (each read once), the step's q/k/v rows, the K/V
    appends and the attention output (bf16)."""
    d, Hq, Hkv = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    row = d * 2
    total, steps = 0, 0
    def step(n_ctx, cols):
        return (2 * Hkv * n_ctx * row + cols * (Hq + 2 * Hkv) * row + cols * 2 * Hkv * row
                + cols * Hq * row)
    for t0 in range(0, p0, chunk):
        T = min(chunk, p0 - t0)
        total += step(t0 + T, T)
        steps += 1
    for i in range(n_new - 1):
        total += step(p0 + i + 1, 1)
        steps += 1
    return total * shape.n_layers, steps * shape.n_layers


_T_START = time.perf_counter()


def progress(msg):
    """One stderr line per finished section (long counter-collection runs)."""
    print("[bench %.1fs] %s" % (time.perf_counter() - _T_START, msg), file=sys.stderr, flush=True)


def run_gpu(args, shape, wl, w, prompt, steps):
    import torch
    from transformer_forward_pass_amd import mak
    m = mak.MakModel(shape, w, device="cuda:0", max_seq=shape.max_seq)
    m.set_prefill_chunk(wl.chunk)
    max_new = wl.max_new
    for _ in range(args.warmup):
        m.generate(prompt, max_new)
    torch.cuda.synchronize()
    progress("%s: warmup done" % shape.name)
    # each step timed on its own as well (median and min of the runs)
    runs = []
    t0 = time.perf_counter()
    for _ in range(steps):
        t_run = time.perf_counter()
        m.generate(prompt, max_new)   # returns after its device-to-host token copy
        runs.append(time.perf_counter() - t_run)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    progress("%s: timed steps done" % shape.name)

    # the prompt alone (chunked prefill + LM head), timed the same way, to
    # separate the steady-state decode rate
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        m.prefill(prompt, want_logits=True)
    torch.cuda.synchronize()
    t_prefill = (time.perf_counter() - t1) / steps
    progress("%s: prefill timing done" % shape.name)

    # second pass with per-launch HIP events on the model's stream
    m.set_phase_timing(True)
    for _ in range(steps):
        m.generate(prompt, max_new)
    times = m.phase_times()
    m.set_phase_timing(False)
    m.free()
    progress("%s: phase timing done" % shape.name)
    return dt, t_prefill, times, runs


def measure(args, name, steps):
    """Throughput, token roofline and dominant-kernel roofline of one workload."""
    from transformer_forward_pass_amd import synth
    wl = synth.WORKLOADS[name]
    if args.max_new:
        import dataclasses
        wl = dataclasses.replace(wl, max_new=args.max_new)
    shape = wl.shape
    w = synth.make_weights(shape)
    prompt = synth.make_prompts(wl)[0]
    dt, t_prefill, times, runs = run_gpu(args, shape, wl, w, prompt, steps)
    p0, n = len(prompt), wl.max_new
    t_decode = (dt / steps - t_prefill) / (n - 1)
    kinds = [k for k in ("qkv", "attn", "o", "gateup", "down", "lmhead") if times[k][1]]
    dom = max(kinds, key=lambda k: times[k][0])
    avg_s = times[dom][0] / times[dom][1] / 1e3
    if dom == "attn":
        tot, launches = _attn_bytes(shape, p0, n, wl.chunk)
        per_launch = tot // launches
    else:
        per_launch = _gemv_bytes(shape, dom)
    achieved = per_launch / avg_s / 1e9
    avg_pos = p0 + (n - 2) / 2.0
    tok_bytes = shape.streamed_weight_bytes() + shape.kv_bytes_per_position() * (avg_pos + 1)
    tok_gbs = tok_bytes / t_decode / 1e9
    return {
        "shape": shape, "w": w, "prompt": prompt, "wl": wl,
        "tok_s": n * steps / dt, "ms_per_step": 1e3 * dt / steps,
        "runs_ms": {"median": round(1e3 * statistics.median(runs), 4), "min": round(1e3 * min(runs), 4),
                    "n": len(runs)},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "bytes_per_launch": per_launch,
                     "avg_launch_us": round(avg_s * 1e6, 3), "launches": times[dom][1]},
        "token_roofline": {"decode_tok_s": round(1.0 / t_decode, 2), "bytes_per_token": int(tok_bytes),
                           "achieved_gbs": round(tok_gbs, 2), "frac": round(tok_gbs / HBM_PEAK_GBS, 4),
                           "prefill_ms": round(t_prefill * 1e3, 4)},
        "phase_ms_per_step": {k: round(v[0] / steps, 4) for k, v in times.items()},
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_run(shape, w, prompt, n_new, threads):
    """The oracle on one prompt: prefill time, then n_new - 1 decode steps."""
    import ctypes
    from oracle import oracle as O
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(threads))
    o = O.Oracle(shape, w, max_len=len(prompt) + n_new + 1)
    t0 = time.perf_counter()
    lg = o.prefill(prompt)
    t1 = time.perf_counter()
    tok = int(np.argmax(lg))
    for i in range(n_new - 1):
        tok = int(np.argmax(o.decode_step(tok, len(prompt) + i)))
    t2 = time.perf_counter()
    return {"threads": int(threads), "prompt_tokens": len(prompt), "prefill_s": round(t1 - t0, 3),
            "decode_steps": n_new - 1, "decode_s": round(t2 - t1, 3),
            "decode_ms_per_token": round(1e3 * (t2 - t1) / max(1, n_new - 1), 2),
            "generated_tok_s": round(n_new / (t2 - t0), 2)}


def cpu_baseline(shape, w, prompt, n_new, w_1b=None):
    """The CPU oracle (untuned) on bounded samples of the benchmark's
    workloads, on this host: the 135M shape with all threads (the reported
    value: generated tokens per second, prefill included) and with one
    thread, and the 1B shape with all threads."""
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    main = _oracle_run(shape, w, prompt, n_new, threads)
    one = _oracle_run(shape, w, prompt[:8], 4, 1)
    detail = {"all_threads": main, "one_thread": one}
    if w_1b is not None:
        from transformer_forward_pass_amd import synth
        wl = synth.WORKLOADS["llama-3.2-1b"]
        detail["1b_all_threads"] = _oracle_run(wl.shape, w_1b, synth.make_prompts(wl)[0][:8], 4, threads)
    import ctypes
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(threads)
    return {"value": main["generated_tok_s"], "unit": "tok/s", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "os_cpu_count": os.cpu_count(),
            "sample": "the %s-shaped model: %d-token prompt then %d greedy tokens on %d threads (value); "
                      "8-token prompt + 4 tokens on 1 thread; the 1B shape: 8-token prompt + 4 tokens on %d "
                      "threads" % (shape.name, len(prompt), n_new, threads, threads),
            "detail": detail}


def measure_batched(args, name="tinyllama-1.1b", reps=2):
    """Batched decode (8 or 16 sequences with their own slots and positions,
    one multi-column step per token): aggregate tok/s over 127 steps after
    each sequence's prompt is prefilled, plus per-phase times and the
    dominant GEMV's roofline over a timed pass of 16 steps."""
    import torch
    from transformer_forward_pass_amd import mak, synth
    wl = synth.WORKLOADS[name]
    shape = wl.shape
    w = synth.make_weights(shape)
    prompts = synth.make_prompts(wl)
    B = len(prompts)
    m = mak.MakModel(shape, w, device="cuda:0", max_seq=shape.max_seq, max_batch=B)
    first = [int(torch.argmax(m.prefill(p, slot=b)).item()) for b, p in enumerate(prompts)]
    pos = [len(p) for p in prompts]
    steps = wl.max_new - 1
    m.decode_batch(first, pos, steps=2, want_logits=False)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(reps):
        ev0.record()
        m.decode_batch(first, pos, steps=steps, want_logits=False)
        ev1.record()
        torch.cuda.synchronize()
        t = ev0.elapsed_time(ev1) / 1e3
        best = t if best is None else min(best, t)
    m.set_phase_timing(True)
    m.decode_batch(first, pos, steps=16, want_logits=False)
    times = m.phase_times()
    m.set_phase_timing(False)
    m.free()
    kinds = [k for k in ("qkv", "o", "gateup", "down", "lmhead") if times[k][1]]
    dom = max(kinds, key=lambda k: times[k][0])
    avg_s = times[dom][0] / times[dom][1] / 1e3
    per_launch = _gemv_bytes(shape, dom)
    avg_ctx = sum(pos) / B + steps / 2.0
    step_bytes = shape.streamed_weight_bytes() + shape.kv_bytes_per_position() * avg_ctx * B
    t_step = best / steps
    return {"workload": "%s-shaped random-init decoder: %d sequences (prompts of %d..%d tokens), "
                        "%d greedy tokens each decoded together" % (name, B, min(pos), max(pos), wl.max_new),
            "value": round(B * steps / best, 2), "unit": "tok/s (all sequences)",
            "ms_per_step": round(t_step * 1e3, 4),
            "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(per_launch / avg_s / 1e9, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(per_launch / avg_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                         "bytes_per_launch": per_launch, "avg_launch_us": round(avg_s * 1e6, 3),
                         "launches": times[dom][1]},
            "step_roofline": {"bytes_per_step": int(step_bytes),
                              "achieved_gbs": round(step_bytes / t_step / 1e9, 2),
                              "frac": round(step_bytes / t_step / 1e9 / HBM_PEAK_GBS, 4)},
            # fp64 rate of the dominant GEMM: 2 flops per weight per sequence
            # (on the fp64 matrix cores or on the vector units, as planned)
            "mfma_roofline": {"bound": "mfma" if _on_matrix_cores(shape, dom, B) else "alu", "kernel": dom,
                              "achieved": round(per_launch / 2 * 2 * B / avg_s / 1e12, 3),
                              "peak": FP64_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s (fp64)",
                              "frac": round(per_launch * B / avg_s / 1e12 / FP64_MFMA_PEAK_TFLOPS, 4)},
            "phase_ms_per_step": {k: round(v[0] / 16, 4) for k, v in times.items()}}


def measure_long(args, name="qwen3-0.6b", reps=2):
    """Long context: a 512-token prompt in 64 chunks of 8 (the workload's
    chunk), then 256 greedy tokens (decode attention runs split-KV past 384
    positions at head_dim 128)."""
    import torch
    from transformer_forward_pass_amd import mak, synth
    wl = synth.WORKLOADS[name]
    shape = wl.shape
    w = synth.make_weights(shape)
    prompt = synth.make_prompts(wl)[0]
    m = mak.MakModel(shape, w, device="cuda:0", max_seq=shape.max_seq)
    m.set_prefill_chunk(wl.chunk)
    m.generate(prompt, 8)
    torch.cuda.synchronize()
    best = bestp = None
    for _ in range(reps):
        t0 = time.perf_counter()
        m.generate(prompt, wl.max_new)
        torch.cuda.synchronize()
        t = time.perf_counter() - t0
        best = t if best is None else min(best, t)
        t0 = time.perf_counter()
        m.prefill(prompt, want_logits=False)
        torch.cuda.synchronize()
        tp = time.perf_counter() - t0
        bestp = tp if bestp is None else min(bestp, tp)
    m.set_phase_timing(True)
    m.generate(prompt, wl.max_new)
    times = m.phase_times()
    m.set_phase_timing(False)
    # the same prompt in chunks of 16 (bitwise the same cache and logits)
    m.set_prefill_chunk(16)
    m.prefill(prompt, want_logits=False)
    torch.cuda.synchronize()
    bestp16 = None
    for _ in range(reps):
        t0 = time.perf_counter()
        m.prefill(prompt, want_logits=False)
        torch.cuda.synchronize()
        tp = time.perf_counter() - t0
        bestp16 = tp if bestp16 is None else min(bestp16, tp)
    m.free()
    t_dec = (best - bestp) / (wl.max_new - 1)
    p0, n = len(prompt), wl.max_new
    avg_ctx = p0 + n / 2.0
    tok_bytes = shape.streamed_weight_bytes() + shape.kv_bytes_per_position() * avg_ctx
    prefill_bytes = (p0 // wl.chunk) * shape.streamed_weight_bytes() * 1.0
    return {"workload": "%s-shaped random-init decoder: %d-token prompt (chunks of %d) + %d greedy tokens, "
                        "batch 1" % (name, p0, wl.chunk, n),
            "value": round(n / best, 2), "unit": "tok/s",
            "decode_tok_s": round(1.0 / t_dec, 2), "prefill_ms": round(bestp * 1e3, 3),
            "token_roofline": {"bytes_per_token": int(tok_bytes),
                               "achieved_gbs": round(tok_bytes / t_dec / 1e9, 2),
                               "frac": round(tok_bytes / t_dec / 1e9 / HBM_PEAK_GBS, 4)},
            "prefill_weight_gbs": round(prefill_bytes / bestp / 1e9, 2),
            "prefill_ms_chunk16": round(bestp16 * 1e3, 3),
            "phase_ms_per_call": {k: round(v[0], 4) for k, v in times.items()}}


FP64_MFMA_PEAK_TFLOPS = 78.6


def measure_long_prefill(args, name="llama-3.2-1b-p2040", reps=2):
    """Long-prompt prefill: a 2040-token prompt on the 1B shape in chunks of
    16 (the GEMMs on the fp64 matrix cores; single-pass attention up to 2048
    positions), and in chunks of 8 for comparison.  Reports the prompt's
    prefill time and the fp64 rate of its weight GEMMs (2 flops per weight
    per token) against the fp64 matrix peak."""
    import torch
    from transformer_forward_pass_amd import mak, synth
    wl = synth.WORKLOADS[name]
    shape = wl.shape
    w = synth.make_weights(shape)
    prompt = synth.make_prompts(wl)[0]
    m = mak.MakModel(shape, w, device="cuda:0", max_seq=shape.max_seq)
    res = {}
    for chunk in (16, 8):
        m.set_prefill_chunk(chunk)
        m.prefill(prompt[:64], want_logits=False)
        torch.cuda.synchronize()
        best = None
        for _ in range(reps if chunk == 16 else 1):
            t0 = time.perf_counter()
            m.prefill(prompt, want_logits=True)
            torch.cuda.synchronize()
            t = time.perf_counter() - t0
            best = t if best is None else min(best, t)
        res[chunk] = best
    m.set_prefill_chunk(16)
    m.set_phase_timing(True)
    m.prefill(prompt, want_logits=True)
    times = m.phase_times()
    m.set_phase_timing(False)
    m.free()
    H, I, qd, kvd = shape.hidden, shape.intermediate, shape.q_dim, shape.kv_dim
    layer_w = H * (qd + 2 * kvd) + qd * H + 3 * H * I
    P = len(prompt)
    gemm_flop = 2.0 * P * shape.n_layers * layer_w + 2.0 * shape.vocab * H
    gemm_s = sum(times[k][0] for k in ("qkv", "o", "gateup", "down", "lmhead")) / 1e3
    achieved = gemm_flop / gemm_s / 1e12
    return {"workload": "%s-shaped random-init decoder: %d-token prompt, chunks of 16" % (shape.name, P),
            "prefill_ms": round(res[16] * 1e3, 3), "prefill_tok_s": round(P / res[16], 1),
            "prefill_ms_chunk8": round(res[8] * 1e3, 3),
            "mfma_roofline": {"bound": "mfma", "kernel": "weight GEMMs (k_gemm16, k_gemm8)", "achieved": round(achieved, 2),
                              "peak": FP64_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s (fp64)",
                              "frac": round(achieved / FP64_MFMA_PEAK_TFLOPS, 4)},
            "phase_ms": {k: round(v[0], 3) for k, v in times.items()}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-new", type=int, default=24, help="greedy tokens of the CPU sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the 1B-shape measurement")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the batched-decode and long-context measurements")
    ap.add_argument("--workload", default=WORKLOAD, choices=[WORKLOAD, SECONDARY, "llama-3.2-1b-mxfp4"],
                    help="batch-1 workload of the main line (the other one goes to `secondary`)")
    ap.add_argument("--max-new", type=int, default=0,
                    help="override the greedy token count (short counter-collection runs only)")
    ap.add_argument("--only", choices=["batched", "batched16", "long_context", "long_prefill"],
                    help="run one of the secondary measurements alone and print its JSON (kernel profiles)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    from transformer_forward_pass_amd import mak
    if not os.path.exists(mak.LIB_PATH):
        from transformer_forward_pass_amd import build as B
        B.build()
    if args.only:
        one = {"batched": lambda: measure_batched(args),
               "batched16": lambda: measure_batched(args, "tinyllama-1.1b-b16"),
               "long_context": lambda: measure_long(args),
               "long_prefill": lambda: measure_long_prefill(args)}[args.only]
        print(json.dumps({args.only: one()}))
        return
    primary = args.workload
    other = SECONDARY if primary == WORKLOAD else WORKLOAD
    r = measure(args, primary, args.steps)
    wl = r["wl"]
    p0, n = len(r["prompt"]), wl.max_new
    r["roofline"]["traffic"] = measured_traffic(r["roofline"]["kernel"])
    out = {
        "metric": "greedy decode tok/s at batch 1 (135M/1B shapes); % of HBM weight-streaming roofline",
        "value": round(r["tok_s"], 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4" if primary.endswith("mxfp4") else "bf16",
        "data": "synthetic",
        "config": {"workload": "%s-shaped random-init decoder: %d-token prompt (chunks of %d) + "
                               "%d greedy tokens, batch 1" % (primary, p0, wl.chunk, n),
                   "accumulate": "f64"},
        "roofline": r["roofline"],
        "token_roofline": r["token_roofline"],
        "phase_ms_per_step": r["phase_ms_per_step"],
        "runs_ms": r["runs_ms"],
    }
    if not args.no_secondary:
        r2 = measure(args, other, max(2, args.steps // 2))
        out["secondary"] = {"workload": "%s-shaped random-init decoder: 32-token prompt (chunks of %d) + "
                                        "128 greedy tokens, batch 1" % (other, r2["wl"].chunk),
                            "value": round(r2["tok_s"], 2), "unit": "tok/s",
                            "ms_per_step": round(r2["ms_per_step"], 4),
                            "roofline": r2["roofline"], "token_roofline": r2["token_roofline"],
                            "phase_ms_per_step": r2["phase_ms_per_step"], "runs_ms": r2["runs_ms"]}
    if not args.no_extra and not args.max_new:
        out["batched"] = measure_batched(args)
        progress("batched decode done")
        out["batched16"] = measure_batched(args, "tinyllama-1.1b-b16")
        progress("16-sequence batched decode done")
        out["long_context"] = measure_long(args)
        progress("long-context run done")
        out["long_prefill"] = measure_long_prefill(args)
        progress("long-prompt prefill done")
        r4 = measure(args, "llama-3.2-1b-mxfp4", max(2, args.steps // 2))
        out["mxfp4"] = {"workload": "llama-3.2-1b-shaped random-init decoder, per-layer linear weights in "
                                    "4-bit OCP MXFP4 (LM head bf16): 32-token prompt (chunks of %d) + "
                                    "128 greedy tokens, batch 1" % r4["wl"].chunk,
                        "value": round(r4["tok_s"], 2), "unit": "tok/s",
                        "dtype": "mxfp4 weights (E2M1 codes, E8M0 scale per 32), bf16 activations, f64 accumulation",
                        "ms_per_step": round(r4["ms_per_step"], 4),
                        "roofline": r4["roofline"], "token_roofline": r4["token_roofline"],
                        "phase_ms_per_step": r4["phase_ms_per_step"], "runs_ms": r4["runs_ms"]}
        progress("4-bit decode done")
    if not args.no_cpu:
        w_1b = r2["w"] if (not args.no_secondary and other == SECONDARY) else None
        out["cpu_baseline"] = cpu_baseline(r["shape"], r["w"], r["prompt"], args.cpu_new, w_1b)
        progress("CPU oracle baseline done")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
