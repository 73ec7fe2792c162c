"""Pins for the oracle's single ops against closed forms, exact integer
arithmetic, textbook identities and brute force.  None of these re-types the
oracle's own formula: each compares against a different route to the same
value."""
import math

import numpy as np
import pytest


def _bf16_ints(rng, shape, lo=-64, hi=64):
    """bf16 bit patterns of small integers (exactly representable)."""
    v = rng.integers(lo, hi + 1, shape).astype(np.float32)
    return v.view(np.uint32).__rshift__(16).astype(np.uint16), v.astype(np.float64)


# ---------------------------------------------------------------- dot / linear

def test_dot_integer_inputs_exact(orc):
    rng = np.random.default_rng(0)
    for K in (1, 7, 64, 576, 4099):
        wb, wv = _bf16_ints(rng, K)
        _, x = _bf16_ints(rng, K)
        exact = sum(int(a) * int(b) for a, b in zip(wv, x))
        assert orc.dot(wb, x) == exact


def test_dot_random_matches_fsum(orc):
    rng = np.random.default_rng(1)
    for K in (64, 1000, 8192):
        w = orc.bf16_from_f32(rng.standard_normal(K).astype(np.float32) * 0.02)
        x = orc.bf16_to_f64(orc.bf16_from_f32(rng.standard_normal(K).astype(np.float32)))
        prods = orc.bf16_to_f64(w) * x            # exact: 8-bit x 8-bit mantissas
        ref = np.float32(math.fsum(prods))        # correctly rounded sum
        assert np.float32(orc.dot(w, x)) == ref


def test_linear_orientation_and_rows(orc):
    """y = W x with W [out, in]: a non-square integer case against integer
    matmul, so a transposed operand or a wrong row stride fails."""
    rng = np.random.default_rng(2)
    N, K, T = 37, 19, 3
    Wb, Wv = _bf16_ints(rng, (N, K), -8, 8)
    _, X = _bf16_ints(rng, (T, K), -8, 8)
    Y = orc.linear(Wb, X, orc.OUT_F64)
    ref = X.astype(np.int64) @ Wv.astype(np.int64).T
    assert np.array_equal(Y, ref.astype(np.float64))
    # output rounding: bf16 of an exact integer sum
    Yb = orc.linear(Wb, X * 37.0, orc.OUT_BF16)
    assert np.array_equal(Yb, orc.round_bf(ref * 37.0))


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_constant_vector_closed_form(orc):
    rng = np.random.default_rng(4)
    n, eps = 96, 1e-5
    w = orc.bf16_from_f32((1 + 0.01 * rng.standard_normal(n)).astype(np.float32))
    for c in (0.75, -3.0, 1e-3):
        out = orc.rmsnorm(np.full(n, c), w, eps, rnd=False)
        ref = orc.bf16_to_f64(w) * (c / math.sqrt(c * c + eps))
        assert np.allclose(out, ref, rtol=1e-15, atol=0)


def test_rmsnorm_unit_weight_mean_square(orc):
    """With w = 1: mean(out^2) = ms / (ms + eps) for any x (fp64 mode)."""
    rng = np.random.default_rng(5)
    n, eps = 576, 1e-3
    w = np.full(n, 0x3F80, np.uint16)        # bf16 1.0
    x = rng.standard_normal(n) * 0.3
    out = orc.rmsnorm(x, w, eps, rnd=False)
    ms = math.fsum(x * x) / n
    assert math.isclose(math.fsum(out * out) / n, ms / (ms + eps), rel_tol=1e-14)


def test_rmsnorm_power_of_four_scale_invariance_bitwise(orc):
    """eps = 0: scaling x by 4^k scales the statistic by exactly 16^k and the
    inverse root by exactly 4^-k, so the rounded output is bitwise unchanged."""
    rng = np.random.default_rng(6)
    n = 256
    w = orc.bf16_from_f32((1 + 0.01 * rng.standard_normal(n)).astype(np.float32))
    x = orc.round_bf(rng.standard_normal(n))
    base = orc.rmsnorm(x, w, 0.0)
    for k in (-3, 1, 4):
        assert np.array_equal(orc.rmsnorm(x * 4.0 ** k, w, 0.0), base)


def test_rmsnorm_rounded_close_to_exact(orc):
    rng = np.random.default_rng(7)
    n = 2048
    w = orc.bf16_from_f32((1 + 0.01 * rng.standard_normal(n)).astype(np.float32))
    x = orc.round_bf(rng.standard_normal(n) * 0.05)
    a = orc.rmsnorm(x, w, 1e-5)
    b = orc.rmsnorm(x, w, 1e-5, rnd=False)
    assert np.all(np.abs(a - b) <= 2 ** -7 * np.abs(b) + 1e-30)   # two bf16 roundings


# --------------------------------------------------------------------- rope

def test_rope_position_zero_is_identity_bitwise(orc):
    rng = np.random.default_rng(8)
    for d in (64, 128):
        u = orc.round_bf(rng.standard_normal(d))
        assert np.array_equal(orc.rope(u, 0, 10000.0), u)
        c, s = orc.rope_table(0, d, 10000.0)
        assert np.all(c == 1.0) and np.all(s == 0.0)


def test_rope_is_complex_rotation_of_half_pairs(orc):
    """fp64 mode: (u_i + i u_{i+d/2}) * exp(i * pos * theta^(-2i/d)) -- the
    rotate-half pairing and the sign of the rotation."""
    rng = np.random.default_rng(9)
    d, theta = 64, 10000.0
    u = rng.standard_normal(d)
    for pos in (1, 7, 513):
        z = (u[:d // 2] + 1j * u[d // 2:]) * np.exp(
            1j * pos * theta ** (-2.0 * np.arange(d // 2) / d))
        out = orc.rope(u, pos, theta, rnd=False)
        assert np.allclose(out[:d // 2], z.real, rtol=0, atol=1e-12)
        assert np.allclose(out[d // 2:], z.imag, rtol=0, atol=1e-12)


def test_rope_preserves_pair_norms_and_relative_position(orc):
    rng = np.random.default_rng(10)
    d, th = 128, 10000.0
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for pos in (3, 100, 767):
        r = orc.rope(q, pos, th, rnd=False)
        pn = lambda v: v[:d // 2] ** 2 + v[d // 2:] ** 2
        assert np.allclose(pn(r), pn(q), rtol=1e-12)
    for m, n in ((10, 3), (700, 650), (5, 5)):
        lhs = orc.rope(q, m, th, rnd=False) @ orc.rope(k, n, th, rnd=False)
        rhs = orc.rope(q, m - n, th, rnd=False) @ k
        assert math.isclose(lhs, rhs, rel_tol=1e-9, abs_tol=1e-9)


def test_rope_rounded_pair_norm_within_bf16(orc):
    rng = np.random.default_rng(11)
    d = 64
    u = orc.round_bf(rng.standard_normal(d))
    for pos in (1, 31, 159):
        r = orc.rope(u, pos, 10000.0)
        n0 = u[:d // 2] ** 2 + u[d // 2:] ** 2
        n1 = r[:d // 2] ** 2 + r[d // 2:] ** 2
        assert np.all(np.abs(np.sqrt(n1) - np.sqrt(n0)) <= 2 ** -6 * np.sqrt(n0) + 1e-30)


# ---------------------------------------------------------------- attention

def test_attention_single_position_returns_v_bitwise(orc):
    rng = np.random.default_rng(12)
    d = 64
    q = orc.round_bf(rng.standard_normal(d))
    K = orc.round_bf(rng.standard_normal((1, d)))
    V = orc.round_bf(rng.standard_normal((1, d)))
    assert np.array_equal(orc.attend(q, K, V, 0.125), V[0])


def test_attention_probabilities_sum_to_one(orc):
    rng = np.random.default_rng(13)
    d, n = 64, 50
    q, K = rng.standard_normal(d), rng.standard_normal((n, d))
    out = orc.attend(q, K, np.ones((n, d)), 0.125, rnd=False)
    assert np.allclose(out, 1.0, rtol=0, atol=1e-14)


def test_attention_identical_keys_give_mean_of_values(orc):
    rng = np.random.default_rng(14)
    d, n = 32, 9
    k = rng.standard_normal(d)
    V = rng.standard_normal((n, d))
    out = orc.attend(rng.standard_normal(d), np.tile(k, (n, 1)), V, 0.2, rnd=False)
    assert np.allclose(out, V.mean(axis=0), rtol=0, atol=1e-14)


def test_attention_brute_force_tiny(orc):
    """Brute force in pure Python on tiny shapes: softmax(q.K * scale) V."""
    rng = np.random.default_rng(15)
    for n, d in ((1, 8), (3, 8), (5, 4)):
        q, K, V = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
        s = [sum(q[i] * K[j][i] for i in range(d)) * 0.3 for j in range(n)]
        e = [math.exp(v - max(s)) for v in s]
        ref = [sum(e[j] * V[j][i] for j in range(n)) / sum(e) for i in range(d)]
        assert np.allclose(orc.attend(q, K, V, 0.3, rnd=False), ref, rtol=1e-13, atol=1e-15)


def test_attention_shift_invariance(orc):
    """Adding the same score offset to every position changes nothing (fp64)."""
    rng = np.random.default_rng(16)
    d, n = 16, 12
    q, K, V = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    # an extra coordinate with q=1 and K=c adds c*scale to every score
    q2 = np.append(q, 1.0)
    K2 = np.hstack([K, np.full((n, 1), 3.7)])
    V2 = np.hstack([V, np.zeros((n, 1))])
    a = orc.attend(q, K, V, 0.25, rnd=False)
    b = orc.attend(q2, K2, V2, 0.25, rnd=False)[:d]
    assert np.allclose(a, b, rtol=0, atol=1e-13)


# ------------------------------------------------------------------- SwiGLU

def test_swiglu_closed_forms(orc):
    g = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    u = np.ones(5)
    out = orc.swiglu(g, u, rnd=False)
    sig1 = 1.0 / (1.0 + math.e ** -1)          # logistic(1) = 0.7310585786300049
    assert out[0] == 0.0
    assert math.isclose(out[1], sig1, rel_tol=1e-15)
    assert math.isclose(out[2], -(1 - sig1), rel_tol=1e-15)   # silu(-x) = silu(x) - x
    assert math.isclose(out[3], 40.0, rel_tol=1e-15)
    assert abs(out[4]) < 1e-15
    # gate and up are not interchangeable: silu is applied to the gate only
    g2, u2 = np.array([2.0]), np.array([-1.0])
    assert math.isclose(orc.swiglu(g2, u2, rnd=False)[0], -2.0 / (1 + math.exp(-2.0)), rel_tol=1e-15)


def test_swiglu_rounded_zero_and_large(orc):
    out = orc.swiglu(np.array([0.0, 64.0]), np.array([3.0, 0.5]))
    assert out[0] == 0.0 and out[1] == 32.0


# ---------------------------------------------------------------- residual / argmax

def test_residual_single_rounding_of_exact_sum(orc):
    x = np.array([1.0, 256.0, 1.0])
    y = np.array([2.0 ** -8, 1.0, 2.0 ** -9])
    # 1 + 2^-8 is a bf16 tie -> 1.0 (even); 257 rounds to 256; 1 + 2^-9 -> 1
    assert list(orc.residual(x, y)) == [1.0, 256.0, 1.0]


def test_argmax_lowest_index_on_ties_brute_force(orc):
    rng = np.random.default_rng(17)
    for _ in range(200):
        v = rng.integers(0, 5, rng.integers(1, 40)).astype(np.float64)
        lst = list(v)
        assert orc.argmax(v) == lst.index(max(lst))
