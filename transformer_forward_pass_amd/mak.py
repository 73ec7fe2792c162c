"""Python binding of libmak.so (ctypes).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI declared in include/mak.h.  PyTorch provides the
device arena (one uint8 tensor) and the stream, nothing else.  There is no
fallback: if libmak.so is missing or no GPU is present, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmak.so")

MAK_OK, MAK_EINVAL, MAK_ERANGE, MAK_ENOMEM, MAK_EDEVICE = 0, -1, -2, -3, -4
MAK_MAX_BATCH = 16
MAK_PREFILL_CHUNK = 16

EXPORTS = ("mak_quantize_mxfp4", "mak_plan", "mak_load", "mak_prefill", "mak_decode_step", "mak_decode_step_static", "mak_generate",
           "mak_decode_batch", "mak_batch_max", "mak_slot_length", "mak_read_kv", "mak_set_executor",
           "mak_set_attention_split", "mak_set_block_attention", "mak_set_prefill_chunk", "mak_set_phase_timing",
           "mak_phase_times", "mak_free", "mak_last_error")
EXEC_GRAPH, EXEC_PHASED = 0, 1
WEIGHT_FORMATS = {"bf16": 0, "mxfp4": 1}
PHASES = ("qkv", "attn", "o", "gateup", "down", "lmhead", "ctl")


class MakError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("mak error %d: %s" % (code, msg))
        self.code = code


class mak_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("tie_embeddings", ctypes.c_int32),
                ("qk_norm", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("max_batch", ctypes.c_int32), ("weight_format", ctypes.c_int32)]


_P16 = ctypes.POINTER(ctypes.c_uint16)


class mak_layer_weights(ctypes.Structure):
    _fields_ = [(n, _P16) for n in ("attn_norm", "wq", "wk", "wv", "wo", "q_norm", "k_norm",
                                    "mlp_norm", "w_gate", "w_up", "w_down")]


class mak_weights(ctypes.Structure):
    _fields_ = [("embed", _P16), ("lm_head", _P16), ("final_norm", _P16),
                ("layers", ctypes.POINTER(mak_layer_weights))]


_lib = None


def lib():
    """Load libmak.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmak.so is not built (run __graft_entry__.build())")
        # torch ships its own HIP runtime under the same soname; load it first
        # so that libmak.so binds to the runtime that owns the device arena
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        P, I32 = ctypes.c_void_p, ctypes.c_int32
        L.mak_quantize_mxfp4.argtypes = [P, ctypes.c_int64, I32, P, P]
        L.mak_quantize_mxfp4.restype = ctypes.c_int
        L.mak_plan.argtypes = [ctypes.POINTER(mak_config), ctypes.POINTER(ctypes.c_size_t)]
        L.mak_load.argtypes = [ctypes.POINTER(mak_config), ctypes.POINTER(mak_weights), P,
                               ctypes.c_size_t, P, ctypes.POINTER(P)]
        L.mak_prefill.argtypes = [P, I32, P, I32, I32, P]
        L.mak_decode_step.argtypes = [P, I32, I32, I32, P, P]
        L.mak_decode_step_static.argtypes = [P, I32, I32, I32, P, P]
        L.mak_generate.argtypes = [P, I32, P, I32, I32, P]
        L.mak_decode_batch.argtypes = [P, I32, P, P, P, I32, P, P]
        L.mak_batch_max.argtypes = [P]
        L.mak_slot_length.argtypes = [P, I32]
        L.mak_read_kv.argtypes = [P, I32, I32, I32, I32, P, P]
        L.mak_set_executor.argtypes = [P, ctypes.c_int]
        L.mak_set_attention_split.argtypes = [P, I32]
        L.mak_set_prefill_chunk.argtypes = [P, I32]
        L.mak_set_block_attention.argtypes = [P, I32]
        L.mak_set_phase_timing.argtypes = [P, ctypes.c_int]
        L.mak_phase_times.argtypes = [P, P, P]
        L.mak_free.argtypes = [P]
        L.mak_free.restype = None
        L.mak_last_error.restype = ctypes.c_char_p
        for n in ("mak_plan", "mak_load", "mak_prefill", "mak_decode_step", "mak_decode_step_static", "mak_generate",
                  "mak_decode_batch", "mak_batch_max", "mak_slot_length", "mak_read_kv", "mak_set_executor",
                  "mak_set_phase_timing", "mak_phase_times"):
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != MAK_OK:
        raise MakError(rc, lib().mak_last_error().decode())


def make_config(shape, max_seq: Optional[int] = None, max_batch: Optional[int] = None) -> mak_config:
    return mak_config(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads,
                      shape.head_dim, shape.intermediate, shape.vocab, shape.rms_eps,
                      shape.rope_theta, int(shape.tie_embeddings), int(shape.qk_norm),
                      int(max_seq if max_seq is not None else shape.max_seq),
                      int(max_batch if max_batch is not None else shape.max_batch),
                      WEIGHT_FORMATS[getattr(shape, "weight_format", "bf16")])


def quantize_mxfp4(w_bits: np.ndarray):
    """mak_quantize_mxfp4 on a [rows, k] uint16 bf16 matrix: returns
    (codes [rows, k/2] uint8, two per byte, low nibble first; E8M0 scales
    [rows, k/32] uint8).  Host only."""
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    rows, k = w.shape
    codes = np.zeros((rows, k // 2), np.uint8)
    scales = np.zeros((rows, max(k // 32, 1)), np.uint8)
    _check(lib().mak_quantize_mxfp4(w.ctypes.data, rows, k, codes.ctypes.data, scales.ctypes.data))
    return codes, scales


def plan(shape, max_seq=None, max_batch=None) -> int:
    cfg = make_config(shape, max_seq, max_batch)
    n = ctypes.c_size_t()
    _check(lib().mak_plan(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def _ptr(a):
    if a is None:
        return None
    assert a.dtype == np.uint16 and a.flags.c_contiguous
    return a.ctypes.data_as(_P16)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class MakModel:
    """A packed model on one GPU (the arena is a torch uint8 tensor)."""

    def __init__(self, shape, weights: dict, device: str = "cuda", max_seq: Optional[int] = None,
                 max_batch: Optional[int] = None, stream=None):
        import torch
        self.shape = shape
        self.cfg = make_config(shape, max_seq, max_batch)
        n = ctypes.c_size_t()
        _check(lib().mak_plan(ctypes.byref(self.cfg), ctypes.byref(n)))
        self.arena_bytes = n.value
        self.device = torch.device(device)
        self.arena = torch.empty(self.arena_bytes, dtype=torch.uint8, device=self.device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        layers = (mak_layer_weights * max(1, shape.n_layers))()
        for i, lw in enumerate(weights["layers"]):
            layers[i] = mak_layer_weights(*[_ptr(lw[k]) for k in (
                "attn_norm", "wq", "wk", "wv", "wo", "q_norm", "k_norm", "mlp_norm",
                "w_gate", "w_up", "w_down")])
        w = mak_weights(_ptr(weights["embed"]), _ptr(weights["lm_head"]),
                        _ptr(weights["final_norm"]), layers)
        handle = ctypes.c_void_p()
        _check(lib().mak_load(ctypes.byref(self.cfg), ctypes.byref(w),
                              ctypes.c_void_p(self.arena.data_ptr()), self.arena_bytes,
                              ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(handle)))
        self.h = handle
        self.vocab = shape.vocab

    # -- API ---------------------------------------------------------------

    def _logits(self, rows: int):
        import torch
        return torch.empty((rows, self.vocab), dtype=torch.float32, device=self.device)

    def decode_step(self, token: int, pos: int, slot: int = 0, want_logits: bool = True):
        """One decode step; returns (fp32 logits [V] on the device or None, next token)."""
        lg = self._logits(1) if want_logits else None
        nxt = ctypes.c_int32()
        _check(lib().mak_decode_step(self.h, slot, int(token), int(pos),
                                     ctypes.c_void_p(lg.data_ptr()) if lg is not None else None,
                                     ctypes.byref(nxt)))
        return (lg[0] if lg is not None else None), nxt.value

    def decode_step_static(self, token: int, pos: int, d_logits, d_next, slot: int = 0):
        """mak_decode_step_static: results into caller-allocated device
        tensors (fp32 [V] logits and one int32, either may be None); the
        call only queues the work on the model's stream."""
        _check(lib().mak_decode_step_static(
            self.h, slot, int(token), int(pos),
            ctypes.c_void_p(d_logits.data_ptr()) if d_logits is not None else None,
            ctypes.c_void_p(d_next.data_ptr()) if d_next is not None else None))

    def prefill(self, ids: Sequence[int], start_pos: int = 0, slot: int = 0,
                want_logits: bool = True):
        a = _i32(ids)
        lg = self._logits(1) if want_logits else None
        _check(lib().mak_prefill(self.h, slot, a.ctypes.data, a.size, int(start_pos),
                                 ctypes.c_void_p(lg.data_ptr()) if lg is not None else None))
        return lg[0] if lg is not None else None

    def generate(self, prompt: Sequence[int], max_new: int, slot: int = 0) -> List[int]:
        a = _i32(prompt)
        out = np.zeros(max_new, np.int32)
        _check(lib().mak_generate(self.h, slot, a.ctypes.data, a.size, int(max_new),
                                  out.ctypes.data))
        return [int(t) for t in out]

    def decode_batch(self, tokens, positions, slots=None, steps: int = 1,
                     want_logits: bool = True):
        """Returns (tokens [steps][B] numpy, fp32 logits [B][V] of the last step or None)."""
        t = _i32(tokens)
        B = t.size
        p = _i32(positions)
        s = _i32(slots if slots is not None else range(B))
        out = np.zeros((steps, B), np.int32)
        lg = self._logits(B) if want_logits else None
        _check(lib().mak_decode_batch(self.h, B, s.ctypes.data, t.ctypes.data, p.ctypes.data,
                                      int(steps), out.ctypes.data,
                                      ctypes.c_void_p(lg.data_ptr()) if lg is not None else None))
        return out, lg

    def batch_max(self) -> int:
        return lib().mak_batch_max(self.h)

    def slot_length(self, slot: int) -> int:
        rc = lib().mak_slot_length(self.h, slot)
        if rc < 0:
            _check(rc)
        return rc

    def read_kv(self, layer: int, slot: int, pos0: int, n: int):
        """Cached K and V values as float64 arrays [n_kv_heads, n, head_dim]."""
        s = self.shape
        k = np.zeros((s.n_kv_heads, n, s.head_dim), np.uint16)
        v = np.zeros_like(k)
        _check(lib().mak_read_kv(self.h, layer, slot, pos0, n, k.ctypes.data, v.ctypes.data))
        f = lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return f(k), f(v)

    def set_executor(self, executor: int):
        """EXEC_GRAPH (captured step graphs) or EXEC_PHASED (one launch per phase)."""
        _check(lib().mak_set_executor(self.h, int(executor)))

    def set_attention_split(self, above: int):
        """Split-KV attention once a step's largest pos + 1 exceeds `above` (0: always)."""
        _check(lib().mak_set_attention_split(self.h, int(above)))

    def set_block_attention(self, on: bool):
        """Blockwise split-KV attention for prompt chunks (on by default)."""
        _check(lib().mak_set_block_attention(self.h, int(on)))

    def set_prefill_chunk(self, tokens: int):
        """Prompt tokens per prefill step (1..16; 8 by default)."""
        _check(lib().mak_set_prefill_chunk(self.h, int(tokens)))

    def set_phase_timing(self, enable: bool):
        _check(lib().mak_set_phase_timing(self.h, int(enable)))

    def phase_times(self) -> dict:
        """{phase: (total ms, launches)} accumulated while timing was on."""
        ms = np.zeros(len(PHASES), np.float64)
        n = np.zeros(len(PHASES), np.int64)
        _check(lib().mak_phase_times(self.h, ms.ctypes.data, n.ctypes.data))
        return {k: (float(ms[i]), int(n[i])) for i, k in enumerate(PHASES)}

    def free(self):
        if getattr(self, "h", None) is not None and self.h.value:
            lib().mak_free(self.h)
            self.h = ctypes.c_void_p()
        self.arena = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
