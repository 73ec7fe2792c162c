"""Write the oracle's reference outputs for the full-size workloads.

Calls only ``oracle/`` (and the shared seeded input generator).  For each
workload it runs greedy generation in the oracle and stores, per sequence:
the prompt, the generated tokens, the oracle's top-2 logit gap at every
step, and at a few sampled steps the fp32 logits at fixed sampled vocabulary
indices plus the 16 largest logits (``<name>.json``).  At three of those
steps it also stores the whole fp32 logit vector [V] of some or all
sequences (``<name>.logits.npz``, key ``s<seq>_t<step>``).  The GPU tests
replay the same token stream (teacher forcing) and compare against these
values.

usage: python tests/golden/make_golden.py [workload ...]
"""
import dataclasses
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import oracle as O                      # noqa: E402
from transformer_forward_pass_amd import synth      # noqa: E402

N_SAMPLE_IDX = 512

# The 16-sequence batched decode is checked over its first 32 tokens: every
# step runs the same 16-column kernels as the benchmark's 128.
GOLDEN_WORKLOADS = dict(synth.WORKLOADS)
GOLDEN_WORKLOADS["tinyllama-1.1b-b16"] = dataclasses.replace(synth.WORKLOADS["tinyllama-1.1b-b16"], max_new=32)


def sample_steps(max_new):
    return sorted({0, 1, 2, max_new // 2, max_new - 1})


def full_steps(name, max_new):
    """Steps whose whole logit vector is stored."""
    if name == "tinyllama-1.1b-b16":
        return [1, 2, max_new - 1]
    return [0, 1, max_new - 1]


def full_seqs(name, n_seqs):
    """Sequences whose whole logit vectors are stored: all of a single-
    sequence workload; four of a batch (both ends of each eight-column
    group)."""
    if n_seqs == 1:
        return [0]
    return sorted({0, 7, 8, n_seqs - 1} & set(range(n_seqs))) if n_seqs > 8 else [0, 3, 4, n_seqs - 1]


def sample_indices(vocab):
    rng = np.random.default_rng(7)
    return sorted(int(i) for i in rng.choice(vocab, size=min(N_SAMPLE_IDX, vocab), replace=False))


def make(name):
    wl = GOLDEN_WORKLOADS[name]
    s = wl.shape
    t0 = time.time()
    w = synth.make_weights(s)
    prompts = synth.make_prompts(wl)
    idx = sample_indices(s.vocab)
    steps = sample_steps(wl.max_new)
    fsteps = full_steps(name, wl.max_new)
    fseqs = full_seqs(name, len(prompts))
    seqs, full = [], {}
    for b, p in enumerate(prompts):
        o = O.Oracle(s, w, max_len=len(p) + wl.max_new)
        toks, gaps, lgs = o.generate(p, wl.max_new, chunk=wl.chunk, keep_logits=True)
        samples = {}
        for st in steps:
            lg = lgs[st]
            top = np.argsort(-lg, kind="stable")[:16]
            samples[str(st)] = {"idx_val": [float(lg[i]) for i in idx],
                                "top_idx": [int(i) for i in top],
                                "top_val": [float(lg[i]) for i in top]}
        if b in fseqs:
            for st in fsteps:
                full["s%d_t%d" % (b, st)] = np.asarray(lgs[st], np.float32)
        seqs.append({"prompt": [int(t) for t in p], "tokens": toks,
                     "gaps": [float(g) for g in gaps], "samples": samples})
        print("%s seq %d/%d done %.1fs" % (name, b + 1, len(prompts), time.time() - t0), flush=True)
    out = {"source": "tests/golden/make_golden.py (oracle/ only)",
           "workload": name, "weights_sha256": synth.weights_digest(w),
           "max_new": wl.max_new, "chunk": wl.chunk, "sample_idx": idx,
           "sample_steps": steps, "full_steps": fsteps, "full_seqs": fseqs, "sequences": seqs}
    path = os.path.join(HERE, name + ".json")
    with open(path, "w") as f:
        json.dump(out, f, separators=(",", ":"))
    if name != "tiny":
        np.savez_compressed(os.path.join(HERE, name + ".logits.npz"), **full)
    print("wrote", path, "%.1fs" % (time.time() - t0), flush=True)


if __name__ == "__main__":
    # tiny: the GPU tests compare it with the oracle run in-process; the
    # stored file is the record of the same run
    for n in (sys.argv[1:] or ["tiny", "smollm2-135m", "llama-3.2-1b", "qwen3-0.6b", "tinyllama-1.1b",
                               "tinyllama-1.1b-b16", "llama-3.2-1b-p2040", "llama-3.2-1b-mxfp4"]):
        make(n)
