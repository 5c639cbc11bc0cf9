"""Pins of the oracle's RMSNorm and of the projection of normalised rows (the
fused norm prologue), each against something other than the oracle itself.

The passage: "#004 the same compiler on Apple's chips", section "Decode" (the
norm run inside the next projection's kernel, bit-identical to the separate
kernels).  Reading: r = 1/sqrt(mean_k x_k^2 + eps), xn_k = x_k r gamma_k.
"""
import numpy as np
import pytest

import oracle
from oracle import tolerance
import synth


def _inputs(M, K, seed):
    X = synth.normal_bf16(95, seed, (M, K), 1.0)
    g = (1.0 + 0.25 * np.random.default_rng(seed).standard_normal(K)).astype(np.float32)
    return X, g


def test_unit_rms_with_unit_gamma_and_zero_eps():
    X, _ = _inputs(4, 1024, 1)
    xn = oracle.rmsnorm(X, np.ones(1024, np.float32), 0.0)
    assert np.allclose(np.mean(xn * xn, axis=1), 1.0, rtol=1e-14, atol=0)


@pytest.mark.parametrize("shift", [-7, -1, 3, 12])
def test_power_of_two_scale_invariance(shift):
    """rmsnorm(2^s x) == rmsnorm(x) exactly with eps = 0 (the sum of squares
    scales by 4^s, its square root by 2^s, all exactly)."""
    X, g = _inputs(3, 520, 2)
    Xs = synth.bf16_from_f32(oracle.bf16_bits_to_f64(X).astype(np.float32) * np.float32(2.0 ** shift))
    assert np.array_equal(oracle.rmsnorm(Xs, g, 0.0), oracle.rmsnorm(X, g, 0.0))


def test_constant_row_closed_form():
    K, a, eps = 64, 1.5, 0.25
    X = synth.bf16_from_f32(np.full((1, K), a, np.float32))
    g = np.linspace(0.5, 2.0, K).astype(np.float32)
    want = a / np.sqrt(a * a + eps) * g.astype(np.float64)
    assert np.allclose(oracle.rmsnorm(X, g, eps)[0], want, rtol=1e-15, atol=0)


def test_projection_against_numpy():
    X, g = _inputs(5, 1024, 3)
    W = synth.normal_bf16(96, 0, (77, 1024), 0.02)
    x = oracle.bf16_bits_to_f64(X)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-6)
    want = (x * r * g.astype(np.float64)) @ oracle.bf16_bits_to_f64(W).T
    got = oracle.rmsnorm_matmul(X, g, W, 1e-6)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    terms = oracle.rmsnorm_matmul(X, g, W, 1e-6, absolute=True)
    assert np.allclose(terms, np.abs(x * r * g.astype(np.float64)) @ np.abs(oracle.bf16_bits_to_f64(W)).T,
                       rtol=1e-12, atol=0)
    assert np.all(terms >= np.abs(got))


def test_gamma_scales_output_linearly():
    X, g = _inputs(2, 256, 4)
    W = synth.normal_bf16(96, 1, (33, 256), 0.02)
    a = oracle.rmsnorm_matmul(X, g, W, 1e-6)
    b = oracle.rmsnorm_matmul(X, (2.0 * g).astype(np.float32), W, 1e-6)
    assert np.array_equal(b, 2.0 * a)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tolerance_accepts_device_like_rounding_and_rejects_mistakes(dtype):
    X, g = _inputs(4, 1024, 5)
    W = synth.normal_bf16(96, 2, (64, 1024), 0.02)
    ref = oracle.rmsnorm_matmul(X, g, W, 1e-6)
    terms = oracle.rmsnorm_matmul(X, g, W, 1e-6, absolute=True)
    # the device's rounding: normalised elements to bf16, then the projection
    xn = oracle.rmsnorm(X, g, 1e-6)
    xb = oracle.round_bf16(xn)
    y = oracle.matmul(xb, W)
    out = oracle.round_bf16(y) if dtype == "bf16" else oracle.round_f32(y)
    assert tolerance.check_norm_projection(out, ref, terms, dtype).ok
    # no norm at all, or no gamma: rejected
    bad = oracle.matmul(X, W)
    bad_out = oracle.round_bf16(bad) if dtype == "bf16" else oracle.round_f32(bad)
    assert not tolerance.check_norm_projection(bad_out, ref, terms, dtype).ok
    nog = oracle.rmsnorm_matmul(X, np.ones(1024, np.float32), W, 1e-6)
    nog_out = oracle.round_bf16(nog) if dtype == "bf16" else oracle.round_f32(nog)
    assert not tolerance.check_norm_projection(nog_out, ref, terms, dtype).ok


def _planted(X, g, eps, k_minus_one=False, eps_outside=False):
    """The normalisation with one planted mistake (a mean over K - 1 terms, or
    epsilon added outside the square root), plain numpy in fp64: what an
    implementation with that mistake would produce."""
    x = oracle.bf16_bits_to_f64(X)
    K = x.shape[1]
    ms = (x * x).sum(axis=1) / (K - 1 if k_minus_one else K)
    r = 1.0 / (np.sqrt(ms) + eps) if eps_outside else 1.0 / np.sqrt(ms + eps)
    return x * r[:, None] * g.astype(np.float64)[None, :]


@pytest.mark.parametrize("K", [520, 1024, 5120, 17408])
def test_boundary_rows_fix_the_rounded_result(K):
    """Row 0 of synth.norm_boundary_case is all ones, so its mean square is
    exactly 1 and each normalised value is gamma_j / sqrt(1 + eps) =
    m_j (1 + 1/(4K)) / sqrt(1 + 1e-6): above the rounding midpoint m_j by a
    relative 1/(4K) - 5e-7, far more than f32 arithmetic can move it, so it
    rounds to the neighbour `hi` for every j.  A mean over K - 1 terms scales it
    by 1/sqrt(K/(K-1)), about 1 - 1/(2K), below every midpoint: every value
    rounds to `lo` instead.  Row 1 (all 2^-10, mean square 2^-20 next to
    eps = 1e-6) moves by far more than a bf16 ulp when epsilon is added outside
    the square root, or is a different constant."""
    eps = 1e-6
    X, g, lo, hi = synth.norm_boundary_case(K)
    got = oracle.round_bf16(oracle.rmsnorm(X, g, eps))
    assert np.array_equal(got[0], hi)
    assert np.array_equal(oracle.round_bf16(_planted(X, g, eps, k_minus_one=True))[0], lo)
    ref1 = oracle.bf16_bits_to_f64(got[1])
    ulp1 = tolerance.bf16_ulp(ref1)
    for wrong in (_planted(X, g, eps, eps_outside=True), _planted(X, g, 1e-5), _planted(X, g, 0.0)):
        w = oracle.bf16_bits_to_f64(oracle.round_bf16(wrong))[1]
        assert np.all(np.abs(w - ref1) > ulp1)
