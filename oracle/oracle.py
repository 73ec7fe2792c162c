"""CPU oracle for the llama-family decoder forward pass.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module.  It shares no code
with the GPU path: the arithmetic lives in ``oracle.c`` (plain loops, fp64
accumulation in ascending index order, bf16 rounding at the op boundaries of
transformers' eager bf16 execution) and this file only sequences those ops in
the order the pages give:

  embedding gather -> per layer [RMSNorm -> Q/K/V -> (qk RMSNorm) -> rope ->
  KV append -> GQA attention -> O projection + residual -> RMSNorm ->
  gate/up -> SwiGLU -> down projection + residual] -> final RMSNorm ->
  LM head (fp32 logits) -> greedy argmax

("model-as-a-kernel", sections API and Method; RMSNorm as in "Building a GPU
compiler from scratch ... (Emmy)", Tensor IR section).

Multi-token forms (chunked prefill, batches) run the same per-row steps; all
rows of one call append their K/V before any of them attends, and a row at
position p attends to positions 0..p of its own sequence.

``rounding=False`` gives the fp64 mode (no bf16/fp32 rounding anywhere), used
by the closed-form checks.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP over output rows;
    no fast-math and no FMA contraction, so the C source's order is kept)."""
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        P, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
        L.orc_bf16_from_f32.argtypes = [P, P, I]
        L.orc_round_bf.argtypes = [P, P, I]
        L.orc_dot.argtypes = [P, P, I]
        L.orc_dot.restype = D
        L.orc_linear.argtypes = [P, I, I, P, I, P, ctypes.c_int, ctypes.c_int]
        L.orc_rmsnorm.argtypes = [P, I, P, D, P, ctypes.c_int]
        L.orc_rope_table.argtypes = [I, I, D, P, P, ctypes.c_int]
        L.orc_rope.argtypes = [P, I, I, D, ctypes.c_int]
        L.orc_attend.argtypes = [P, P, P, I, I, I, D, P, P, ctypes.c_int]
        L.orc_swiglu.argtypes = [P, P, I, P, ctypes.c_int]
        L.orc_residual.argtypes = [P, P, I, ctypes.c_int]
        L.orc_argmax.argtypes = [P, I]
        L.orc_argmax.restype = I
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _u16(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint16)


# --------------------------------------------------------------------------
# single ops (thin wrappers; the arithmetic is in oracle.c)
# --------------------------------------------------------------------------

def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_from_f32(_p(x), _p(out), x.size)
    return out


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns."""
    b = _u16(b)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf(x: np.ndarray) -> np.ndarray:
    x = _f64(x)
    out = np.empty_like(x)
    lib().orc_round_bf(_p(x), _p(out), x.size)
    return out


def dot(w: np.ndarray, x: np.ndarray) -> float:
    w, x = _u16(w), _f64(x)
    assert w.size == x.size
    return lib().orc_dot(_p(w), _p(x), w.size)


OUT_F64, OUT_F32, OUT_BF16 = 0, 1, 2


def linear(W: np.ndarray, X: np.ndarray, out_mode: int = OUT_BF16, rnd: bool = True) -> np.ndarray:
    """Y[t, i] = round(sum_k W[i, k] X[t, k]) for W [N, K] bf16 bits, X [T, K]."""
    W = _u16(W)
    X = _f64(X)
    squeeze = X.ndim == 1
    X2 = X.reshape(-1, W.shape[1])
    Y = np.empty((X2.shape[0], W.shape[0]), np.float64)
    lib().orc_linear(_p(W), W.shape[0], W.shape[1], _p(X2), X2.shape[0], _p(Y),
                     out_mode, int(rnd))
    return Y[0] if squeeze else Y


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float, rnd: bool = True) -> np.ndarray:
    x, w = _f64(x), _u16(w)
    assert x.size == w.size
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), x.size, _p(w), eps, _p(out), int(rnd))
    return out


def rope_table(pos: int, d: int, theta: float, rnd: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    c = np.empty(d // 2)
    s = np.empty(d // 2)
    lib().orc_rope_table(pos, d, theta, _p(c), _p(s), int(rnd))
    return c, s


def rope(u: np.ndarray, pos: int, theta: float, rnd: bool = True) -> np.ndarray:
    u = _f64(u).copy()
    assert u.size <= 1024 and u.size % 2 == 0
    lib().orc_rope(_p(u), u.size, pos, theta, int(rnd))
    return u


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, rnd: bool = True) -> np.ndarray:
    """One query head over n positions: K, V are [n, d] (rows may be strided
    views of a cache; they are copied contiguous here)."""
    q, K, V = _f64(q), _f64(K), _f64(V)
    n, d = K.shape
    o = np.empty(d)
    work = np.empty(max(n, 1))
    lib().orc_attend(_p(q), _p(K), _p(V), n, d, d, scale, _p(o), _p(work), int(rnd))
    return o


def swiglu(g: np.ndarray, u: np.ndarray, rnd: bool = True) -> np.ndarray:
    g, u = _f64(g), _f64(u)
    m = np.empty_like(g)
    lib().orc_swiglu(_p(g), _p(u), g.size, _p(m), int(rnd))
    return m


def residual(x: np.ndarray, y: np.ndarray, rnd: bool = True) -> np.ndarray:
    x, y = _f64(x).copy(), _f64(y)
    lib().orc_residual(_p(x), _p(y), x.size, int(rnd))
    return x


def argmax(v: np.ndarray) -> int:
    v = _f64(v)
    return int(lib().orc_argmax(_p(v), v.size))


def top2_gap(v: np.ndarray) -> float:
    """Gap between the largest and second largest logit."""
    s = np.sort(np.asarray(v, np.float64))
    return float(s[-1] - s[-2])


# --------------------------------------------------------------------------
# the model
# --------------------------------------------------------------------------

class Oracle:
    """Plain forward pass over a KV cache.

    ``shape`` provides n_layers, hidden, n_q_heads, n_kv_heads, head_dim,
    intermediate, vocab, rms_eps, rope_theta, tie_embeddings, qk_norm.
    ``weights`` is ``{"embed", "lm_head" or None, "final_norm", "layers"}``
    of uint16 bf16 bit arrays in ``[out, in]`` layout.  A shape whose
    ``weight_format`` is ``"mxfp4"`` runs on the dequantized 4-bit form of the
    per-layer linear matrices (``mxfp4.py``), which are exactly bf16 values.
    """

    def __init__(self, shape, weights, *, rounding: bool = True, max_len: int = 2048,
                 n_seqs: int = 1):
        self.s = shape
        if getattr(shape, "weight_format", "bf16") == "mxfp4":
            from . import mxfp4
            weights = mxfp4.dequantized_weights(shape, weights)
        self.w = weights
        self.rnd = bool(rounding)
        self.max_len = int(max_len)
        L, Hkv, d = shape.n_layers, shape.n_kv_heads, shape.head_dim
        self.K = [[np.zeros((Hkv, self.max_len, d)) for _ in range(L)] for _ in range(n_seqs)]
        self.V = [[np.zeros((Hkv, self.max_len, d)) for _ in range(L)] for _ in range(n_seqs)]
        self.lm = weights["embed"] if shape.tie_embeddings else weights["lm_head"]

    # -- steps -------------------------------------------------------------

    def _norm_rows(self, X: np.ndarray, w: np.ndarray) -> np.ndarray:
        return np.stack([rmsnorm(x, w, self.s.rms_eps, self.rnd) for x in X])

    def _attention_block(self, l: int, X: np.ndarray, rows) -> np.ndarray:
        s, lw, rnd = self.s, self.w["layers"][l], self.rnd
        d, Hq, Hkv = s.head_dim, s.n_q_heads, s.n_kv_heads
        Hn = self._norm_rows(X, lw["attn_norm"])
        Q = linear(lw["wq"], Hn, OUT_BF16, rnd).reshape(len(rows), Hq, d)
        Kx = linear(lw["wk"], Hn, OUT_BF16, rnd).reshape(len(rows), Hkv, d)
        Vx = linear(lw["wv"], Hn, OUT_BF16, rnd).reshape(len(rows), Hkv, d)
        for t, (seq, _, pos) in enumerate(rows):
            for h in range(Hq):
                if s.qk_norm:
                    Q[t, h] = rmsnorm(Q[t, h], lw["q_norm"], s.rms_eps, rnd)
                Q[t, h] = rope(Q[t, h], pos, s.rope_theta, rnd)
            for g in range(Hkv):
                if s.qk_norm:
                    Kx[t, g] = rmsnorm(Kx[t, g], lw["k_norm"], s.rms_eps, rnd)
                Kx[t, g] = rope(Kx[t, g], pos, s.rope_theta, rnd)
                self.K[seq][l][g, pos] = Kx[t, g]
                self.V[seq][l][g, pos] = Vx[t, g]
        # every row of the call has appended its K/V before any row attends
        O = np.empty((len(rows), Hq * d))
        group = Hq // Hkv
        scale = 1.0 / np.sqrt(float(d))
        for t, (seq, _, pos) in enumerate(rows):
            for h in range(Hq):
                g = h // group
                O[t, h * d:(h + 1) * d] = attend(Q[t, h], self.K[seq][l][g, :pos + 1],
                                                 self.V[seq][l][g, :pos + 1], scale, rnd)
        Y = linear(lw["wo"], O, OUT_BF16, rnd)
        return np.stack([residual(X[t], Y[t], rnd) for t in range(len(rows))])

    def _mlp_block(self, l: int, X: np.ndarray) -> np.ndarray:
        lw, rnd = self.w["layers"][l], self.rnd
        H2 = self._norm_rows(X, lw["mlp_norm"])
        G = linear(lw["w_gate"], H2, OUT_BF16, rnd)
        U = linear(lw["w_up"], H2, OUT_BF16, rnd)
        M = np.stack([swiglu(G[t], U[t], rnd) for t in range(len(X))])
        D = linear(lw["w_down"], M, OUT_BF16, rnd)
        return np.stack([residual(X[t], D[t], rnd) for t in range(len(X))])

    def hidden(self, rows: Sequence[Tuple[int, int, int]]) -> np.ndarray:
        """Run rows (seq, token, pos) through every layer; returns X [T, H]."""
        rows = list(rows)
        for seq, tok, pos in rows:
            if not (0 <= tok < self.s.vocab) or not (0 <= pos < self.max_len):
                raise ValueError("token or position out of range")
        X = np.stack([bf16_to_f64(self.w["embed"][tok]) for _, tok, _ in rows])
        for l in range(self.s.n_layers):
            X = self._attention_block(l, X, rows)
            X = self._mlp_block(l, X)
        return X

    def logits_of(self, x: np.ndarray) -> np.ndarray:
        """fp32 logits (as float64 holding fp32 values) of one final hidden row."""
        hf = rmsnorm(x, self.w["final_norm"], self.s.rms_eps, self.rnd)
        return linear(self.lm, hf, OUT_F32, self.rnd)

    def forward(self, rows, want_logits: Optional[Sequence[bool]] = None) -> List[Optional[np.ndarray]]:
        rows = list(rows)
        X = self.hidden(rows)
        if want_logits is None:
            want_logits = [True] * len(rows)
        return [self.logits_of(X[t]) if want_logits[t] else None for t in range(len(rows))]

    # -- API-shaped helpers ------------------------------------------------

    def decode_step(self, token: int, pos: int, seq: int = 0) -> np.ndarray:
        return self.forward([(seq, token, pos)])[0]

    def prefill(self, ids, start_pos: int = 0, seq: int = 0, chunk: int = 8) -> np.ndarray:
        """Consume ids in chunks of at most `chunk` tokens starting at
        start_pos; logits of the last token only."""
        ids = [int(t) for t in ids]
        out = None
        for c0 in range(0, len(ids), chunk):
            part = ids[c0:c0 + chunk]
            rows = [(seq, t, start_pos + c0 + i) for i, t in enumerate(part)]
            last = c0 + chunk >= len(ids)
            res = self.forward(rows, [last and i == len(part) - 1 for i in range(len(part))])
            if last:
                out = res[-1]
        return out

    def generate(self, prompt, max_new: int, seq: int = 0, chunk: int = 8,
                 keep_logits: bool = False):
        """Greedy generation: max_new tokens, the first from the prefill
        logits.  Returns (tokens, top-2 gaps, logits list or None)."""
        prompt = [int(t) for t in prompt]
        lg = self.prefill(prompt, 0, seq, chunk)
        toks, gaps, lgs = [], [], []
        pos = len(prompt)
        for i in range(max_new):
            t = argmax(lg)
            toks.append(t)
            gaps.append(top2_gap(lg))
            if keep_logits:
                lgs.append(lg)
            if i + 1 < max_new:
                lg = self.decode_step(t, pos, seq)
                pos += 1
        return toks, gaps, (lgs if keep_logits else None)
