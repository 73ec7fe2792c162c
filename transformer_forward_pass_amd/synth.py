"""Seeded synthetic inputs: model shapes, random-init bf16 weights and prompts.

This module is the single input generator shared by the GPU path's tests and
benchmark and by the CPU oracle's tests.  It holds none of the forward pass's
arithmetic: it only draws random numbers and stores them as bf16 bit patterns.

Shapes follow the checkpoints measured on the "model-as-a-kernel" page
(section "Measured": SmolLM2-135M, Llama-3.2-1B) and the families its API
section lists as supported (Qwen3 dense with qk RMSNorm, TinyLlama).  The
trained checkpoints are not available, so every model here is random-init:

* linear weights  = bf16(f32(z * 0.02)),       z ~ N(0, 1) drawn as float32
* norm weights    = bf16(f32(1 + f32(z * 0.01)))
* draw order      = embed; per layer attn_norm, wq, wk, wv, [q_norm, k_norm],
                    wo, mlp_norm, w_gate, w_up, w_down; final_norm; lm_head
                    (only when untied)
* weights seed 0, prompt seed 1 (numpy ``default_rng``); prompt ids uniform.

Weight matrices use the ``[out, in]`` row-major layout of a linear layer.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List

import numpy as np


@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    tie_embeddings: bool = False
    qk_norm: bool = False
    max_seq: int = 2048
    max_batch: int = 1
    weight_format: str = "bf16"   # per-layer linear matrices: "bf16" or "mxfp4" (4-bit)

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def n_params(self) -> int:
        H, I = self.hidden, self.intermediate
        per_layer = (H * (self.q_dim + 2 * self.kv_dim) + self.q_dim * H
                     + 3 * H * I + 2 * H)
        if self.qk_norm:
            per_layer += 2 * self.head_dim
        n = self.vocab * H + self.n_layers * per_layer + H
        if not self.tie_embeddings:
            n += self.vocab * H
        return n

    def streamed_weight_bytes(self) -> int:
        """Bytes one decode token must read once: every layer weight, the
        final norm and the LM head (the embedding row itself is 2*H).  With
        4-bit weights each linear weight takes half a byte plus one scale
        byte per 32 weights; norms and the LM head stay bf16."""
        H, I = self.hidden, self.intermediate
        lin = H * (self.q_dim + 2 * self.kv_dim) + self.q_dim * H + 3 * H * I
        norms = 2 * H + (2 * self.head_dim if self.qk_norm else 0)
        lin_bytes = lin // 2 + lin // 32 if self.weight_format == "mxfp4" else 2 * lin
        return self.n_layers * (lin_bytes + 2 * norms) + 2 * (H + self.vocab * H + H)

    def kv_bytes_per_position(self) -> int:
        """K and V bytes of one cached position over all layers (bf16)."""
        return 2 * 2 * self.n_layers * self.kv_dim


@dataclasses.dataclass(frozen=True)
class Workload:
    """A decode recipe: prompt length(s), tokens generated, batch, chunk."""
    shape: ModelShape
    prompt_len: int          # for batched workloads: lower bound of the length draw
    max_new: int
    batch: int = 1
    prompt_len_hi: int = 0   # batched workloads draw lengths uniform in [prompt_len, hi]
    chunk: int = 8


SHAPES: Dict[str, ModelShape] = {
    "tiny": ModelShape("tiny", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2,
                       head_dim=64, intermediate=688, vocab=4096),
    "smollm2-135m": ModelShape("smollm2-135m", n_layers=30, hidden=576, n_q_heads=9,
                               n_kv_heads=3, head_dim=64, intermediate=1536,
                               vocab=49152, tie_embeddings=True),
    "llama-3.2-1b": ModelShape("llama-3.2-1b", n_layers=16, hidden=2048, n_q_heads=32,
                               n_kv_heads=8, head_dim=64, intermediate=8192,
                               vocab=128256, tie_embeddings=True),
    "qwen3-0.6b": ModelShape("qwen3-0.6b", n_layers=28, hidden=1024, n_q_heads=16,
                             n_kv_heads=8, head_dim=128, intermediate=3072,
                             vocab=151936, tie_embeddings=True, qk_norm=True),
    "tinyllama-1.1b": ModelShape("tinyllama-1.1b", n_layers=22, hidden=2048,
                                 n_q_heads=32, n_kv_heads=4, head_dim=64,
                                 intermediate=5632, vocab=32000, max_batch=8),
}

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(SHAPES["tiny"], prompt_len=16, max_new=32),
    # the 32 + 128 batch-1 workloads: the prompt in two chunks of 16
    "smollm2-135m": Workload(SHAPES["smollm2-135m"], prompt_len=32, max_new=128, chunk=16),
    "llama-3.2-1b": Workload(SHAPES["llama-3.2-1b"], prompt_len=32, max_new=128, chunk=16),
    "qwen3-0.6b": Workload(SHAPES["qwen3-0.6b"], prompt_len=512, max_new=256),
    "tinyllama-1.1b": Workload(SHAPES["tinyllama-1.1b"], prompt_len=16, max_new=128,
                               batch=8, prompt_len_hi=256),
    # the same shape and weights, 16 sequences decoded together
    "tinyllama-1.1b-b16": Workload(dataclasses.replace(SHAPES["tinyllama-1.1b"], max_batch=16),
                                   prompt_len=16, max_new=128, batch=16, prompt_len_hi=256),
    # long-prompt prefill: a 2040-token prompt on the 1B shape, in chunks of 16
    "llama-3.2-1b-p2040": Workload(SHAPES["llama-3.2-1b"], prompt_len=2040, max_new=4, chunk=16),
    # 4-bit (MXFP4) per-layer weights quantized from the same bf16 weights
    "llama-3.2-1b-mxfp4": Workload(dataclasses.replace(SHAPES["llama-3.2-1b"], name="llama-3.2-1b-mxfp4",
                                                       weight_format="mxfp4"), prompt_len=32, max_new=128,
                                 chunk=16),
}

LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo",
              "mlp_norm", "w_gate", "w_up", "w_down")


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest even) and return the
    16-bit patterns as uint16.  Uses torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _linear(rng: np.random.Generator, shape) -> np.ndarray:
    z = rng.standard_normal(shape, dtype=np.float32)
    z *= np.float32(0.02)
    return bf16_bits(z)


def _norm(rng: np.random.Generator, n: int) -> np.ndarray:
    z = rng.standard_normal(n, dtype=np.float32)
    z *= np.float32(0.01)
    z += np.float32(1.0)
    return bf16_bits(z)


def make_weights(shape: ModelShape, seed: int = 0) -> dict:
    """Random-init weights as uint16 bf16 bit patterns, ``[out, in]`` layout.

    Returns ``{"embed", "lm_head" (None if tied), "final_norm", "layers": [..]}``
    where each layer is a dict keyed by ``LAYER_KEYS`` (q_norm/k_norm None
    unless the shape has qk-norm)."""
    rng = np.random.default_rng(seed)
    H, d = shape.hidden, shape.head_dim
    w = {"embed": _linear(rng, (shape.vocab, H)), "layers": []}
    for _ in range(shape.n_layers):
        lw = {"attn_norm": _norm(rng, H),
              "wq": _linear(rng, (shape.q_dim, H)),
              "wk": _linear(rng, (shape.kv_dim, H)),
              "wv": _linear(rng, (shape.kv_dim, H))}
        if shape.qk_norm:
            lw["q_norm"] = _norm(rng, d)
            lw["k_norm"] = _norm(rng, d)
        else:
            lw["q_norm"] = None
            lw["k_norm"] = None
        lw["wo"] = _linear(rng, (H, shape.q_dim))
        lw["mlp_norm"] = _norm(rng, H)
        lw["w_gate"] = _linear(rng, (shape.intermediate, H))
        lw["w_up"] = _linear(rng, (shape.intermediate, H))
        lw["w_down"] = _linear(rng, (H, shape.intermediate))
        w["layers"].append(lw)
    w["final_norm"] = _norm(rng, H)
    w["lm_head"] = None if shape.tie_embeddings else _linear(rng, (shape.vocab, H))
    return w


def make_prompts(wl: Workload, seed: int = 1) -> List[np.ndarray]:
    """Uniform random prompt ids (int32).  Batched workloads first draw the
    ``batch`` lengths uniform in ``[prompt_len, prompt_len_hi]``."""
    rng = np.random.default_rng(seed)
    if wl.batch > 1:
        lens = rng.integers(wl.prompt_len, wl.prompt_len_hi + 1, wl.batch)
    else:
        lens = [wl.prompt_len]
    return [rng.integers(0, wl.shape.vocab, int(n)).astype(np.int32) for n in lens]


def weights_digest(w: dict) -> str:
    """sha256 over every weight array in draw order (detects generator drift)."""
    h = hashlib.sha256()
    def upd(a):
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    upd(w["embed"])
    for lw in w["layers"]:
        for k in LAYER_KEYS:
            upd(lw[k])
    upd(w["final_norm"])
    upd(w["lm_head"])
    return h.hexdigest()


def small_shape(**kw) -> ModelShape:
    """A tiny shape for unit tests; keyword overrides on top of 'tiny'."""
    return dataclasses.replace(SHAPES["tiny"], **kw)
