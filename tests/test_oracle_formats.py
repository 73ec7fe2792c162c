"""Pins for the oracle's number formats: fp32 -> bf16 round-to-nearest-even.

The rounding helper is checked against torch's CPU cast (an independent
implementation) on every fp32 exponent/sign with the bit patterns around
each rounding boundary, plus random patterns, and on hand-made ties."""
import numpy as np
import torch


def _torch_bf16(f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(f32)
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_cast(orc):
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000],
                    dtype=np.uint32)
    rng = np.random.default_rng(5)
    lows = np.concatenate([lows, rng.integers(0, 1 << 16, 24).astype(np.uint32)])
    bits = (hi[:, None] | lows[None, :]).ravel()
    f = bits.view(np.float32)
    ours = orc.bf16_from_f32(f)
    ref = _torch_bf16(f)
    nan = np.isnan(f)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN (payload may differ)
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x007F) != 0)


def test_bf16_ties_to_even(orc):
    # 1 + 2^-8 is exactly halfway between 1 and 1 + 2^-7: ties go to the even (1.0)
    f = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -20],
                 dtype=np.float32)
    out = orc.bf16_to_f64(orc.bf16_from_f32(f))
    assert list(out) == [1.0, 1 + 2 * 2.0 ** -7, -1.0, 1 + 2.0 ** -7]


def test_round_bf_is_double_rounding_through_fp32(orc):
    # rbf(v) = bf16(fp32(v)): v = 1 + 2^-8 + 2^-30 rounds to fp32 1 + 2^-8 (a bf16
    # tie) and then to 1.0, while a single rounding of v would give 1 + 2^-7.
    v = np.array([1 + 2.0 ** -8 + 2.0 ** -30, 3.0, -0.0, 65504.0])
    assert list(orc.round_bf(v)) == [1.0, 3.0, 0.0, 65536.0]


def test_bf16_exact_values_roundtrip(orc):
    rng = np.random.default_rng(3)
    b = rng.integers(0, 1 << 16, 4096).astype(np.uint16)
    b = b[(b & 0x7F80) != 0x7F80]          # drop inf/NaN
    v = orc.bf16_to_f64(b)
    assert np.array_equal(orc.round_bf(v), v)
