"""CPU reference of the 4-bit weight format: OCP MXFP4.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module.  It shares no code
with the GPU library's quantizer.

The "model-as-a-kernel" page lists 4-bit (bitsandbytes nf4) weights among the
supported variants (API section, "Supported" paragraph) but gives neither the
nf4 code book nor its block layout.  The 4-bit format here is the open one
that gfx950 converts natively: MXFP4 of the OCP Microscaling Formats (MX)
specification v1.0.  A block of 32 consecutive weights of one row shares one
E8M0 scale X = 2^e (e in [-127, 127]); each weight is an FP4 E2M1 element
(sign, 2 exponent bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1,
1.5, 2, 3, 4, 6; no infinities or NaN).  Conversion of a block of scalars,
as the specification describes it:

1. e = floor(log2(max_i |v_i|)) - 2, where 2 is the exponent of E2M1's
   largest normal (6 = 1.5 * 2^2), clamped to E8M0's range [-127, 127];
   a block of zeros takes e = -127.
2. each element is v_i / X rounded to the nearest E2M1 value, ties to the
   value with an even mantissa bit, and magnitudes beyond 6 saturate to 6.

Readings where the specification leaves a choice: saturation (rather than an
error) for magnitudes above 6, the scale of an all-zero block, zero always
encoded with a clear sign bit, and two codes per byte with the element of
lower index in the low nibble.

Every dequantized weight code * 2^e is a value with at most two significant
bits and magnitude in [2^-128, 1.5 * 2^127], so it is exactly a bf16 value:
the oracle runs a 4-bit model as the bf16 model whose linear weights are the
dequantized ones, and its arithmetic is otherwise unchanged.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
# E2M1 magnitudes indexed by the 3 low code bits (exponent bits, mantissa bit)
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E_MAX_ELEM = 2
SCALE_BIAS = 127


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _f64_to_bf16_exact(v: np.ndarray) -> np.ndarray:
    """bf16 bits of values that are exactly bf16 (checked)."""
    f = v.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v), "value not representable in float32"
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


def shared_exponent(block: np.ndarray) -> int:
    """Step 1: the block's scale exponent e (X = 2^e)."""
    amax = float(np.max(np.abs(block)))
    if amax == 0.0:
        return -SCALE_BIAS
    _, ex = np.frexp(amax)             # amax = f * 2^ex, f in [0.5, 1)
    e = int(ex) - 1 - E_MAX_ELEM       # floor(log2(amax)) - 2
    return min(max(e, -SCALE_BIAS), SCALE_BIAS)


def nearest_e2m1(q: float) -> int:
    """Step 2 for one scaled element: the 4-bit code of the E2M1 value nearest
    to q (brute force over the eight magnitudes), ties to the even mantissa
    bit, saturating at 6."""
    a = abs(q)
    best = 0
    for i in range(1, 8):
        d, db = abs(a - E2M1[i]), abs(a - E2M1[best])
        if d < db or (d == db and (i & 1) == 0 and (best & 1) == 1):
            best = i
    sign = 8 if (q < 0 and best != 0) else 0
    return sign | best


def quantize(w_bits: np.ndarray, rows_per_pass: int = 256):
    """[N, K] bf16 bits (K a multiple of 32) -> (codes [N, K] uint8 in 0..15,
    scale exponents [N, K/32] int).  The same two steps as shared_exponent()
    and nearest_e2m1(), applied to whole arrays (rows_per_pass rows at a
    time) so that billion-weight models convert in minutes."""
    w_all = np.ascontiguousarray(w_bits, dtype=np.uint16)
    N, K = w_all.shape
    assert K % BLOCK == 0, "K must be a multiple of 32"
    codes = np.zeros((N, K), np.uint8)
    exps = np.zeros((N, K // BLOCK), np.int64)
    even = (np.arange(8) & 1) == 0
    for r0 in range(0, N, rows_per_pass):
        w = _bf16_to_f64(w_all[r0:r0 + rows_per_pass])
        assert np.all(np.isfinite(w)), "weights must be finite"
        n = w.shape[0]
        blk = w.reshape(n, K // BLOCK, BLOCK)
        amax = np.abs(blk).max(axis=2)
        _, ex = np.frexp(amax)
        e = np.clip(ex.astype(np.int64) - 1 - E_MAX_ELEM, -SCALE_BIAS, SCALE_BIAS)
        e[amax == 0.0] = -SCALE_BIAS
        q = blk / np.power(2.0, e.astype(np.float64))[:, :, None]
        d = np.abs(np.abs(q)[..., None] - E2M1)             # distance to each magnitude
        cand = d == d.min(axis=3, keepdims=True)
        even_cand = cand & even
        idx = np.where(even_cand.any(axis=3), even_cand.argmax(axis=3), cand.argmax(axis=3))
        sign = np.where((q < 0) & (idx != 0), 8, 0)
        codes[r0:r0 + n] = (sign | idx).reshape(n, K).astype(np.uint8)
        exps[r0:r0 + n] = e
    return codes, exps


def dequantize(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """Codes and scale exponents -> [N, K] float64 values."""
    mag = E2M1[codes & 7]
    sgn = np.where(codes & 8, -1.0, 1.0)
    X = np.repeat(np.power(2.0, exps.astype(np.float64)), BLOCK, axis=1)
    return sgn * mag * X


def quantize_dequantize_bf16(w_bits: np.ndarray) -> np.ndarray:
    """The bf16 bits of the dequantized 4-bit weights."""
    codes, exps = quantize(w_bits)
    return _f64_to_bf16_exact(dequantize(codes, exps))


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """[N, K] codes -> [N, K/2] bytes, element 2i in the low nibble."""
    c = codes.astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def scale_bytes(exps: np.ndarray) -> np.ndarray:
    """E8M0 encoding of the scale exponents (e + 127)."""
    return (exps + SCALE_BIAS).astype(np.uint8)


def dequantized_weights(shape, w: dict) -> dict:
    """A weight dict (synth.make_weights layout) with every per-layer linear
    matrix replaced by its dequantized 4-bit form; the embedding, LM head and
    norm weights stay bf16."""
    out = dict(w)
    out["layers"] = []
    for lw in w["layers"]:
        nl = dict(lw)
        for k in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            nl[k] = quantize_dequantize_bf16(lw[k])
        out["layers"].append(nl)
    return out
