"""Pins of the oracle's SwiGLU (the fused gate_up epilogue) and of its
tolerance rule, each against something other than the oracle itself.

The passage: "#004 the same compiler on Apple's chips", section "Decode"
(the SwiGLU folded into the gate_up projection; the fused result keeps the
bits of the separate kernels).  Reading of the layout: gate rows first, then
up rows; silu(g) = g * sigmoid(g) = g / (1 + e^-g).
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import tolerance
import synth


def _gu(M, half, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((M, half)) * 3.0, rng.standard_normal((M, half)) * 2.0


def test_zero_gate_gives_zero():
    g = np.zeros((2, 5))
    u = np.arange(10.0).reshape(2, 5)
    assert np.all(oracle.swiglu(np.hstack([g, u])) == 0.0)


def test_large_gate_passes_up_times_gate():
    g = np.full((1, 4), 40.0)                      # sigmoid(40) = 1 - 4e-18
    u = np.array([[1.0, -2.0, 0.5, 3.0]])
    assert np.allclose(oracle.swiglu(np.hstack([g, u])), g * u, rtol=1e-15, atol=0)


def test_large_negative_gate_vanishes():
    g = np.full((1, 3), -800.0)                    # exp(800) overflows to inf: g / inf = -0
    u = np.array([[1.0, 2.0, 3.0]])
    h = oracle.swiglu(np.hstack([g, u]))
    assert np.all(h == 0.0)


def test_closed_form_at_log3():
    # sigmoid(ln 3) = 3/4 exactly in R, so silu(ln 3) * u = 0.75 ln 3 u
    g = np.array([[math.log(3.0)]])
    u = np.array([[5.0]])
    assert oracle.swiglu(np.hstack([g, u]))[0, 0] == pytest.approx(0.75 * math.log(3.0) * 5.0, rel=1e-15)


def test_reflection_identity():
    # silu(-g) = silu(g) - g, hence swiglu(-g, u) = swiglu(g, u) - g u
    g, u = _gu(3, 64, 1)
    a = oracle.swiglu(np.hstack([-g, u]))
    b = oracle.swiglu(np.hstack([g, u])) - g * u
    assert np.allclose(a, b, rtol=0, atol=1e-12 * (np.abs(g * u).max() + 1))


def test_against_scipy_expit():
    g, u = _gu(4, 257, 2)
    want = g * expit(g) * u
    assert np.allclose(oracle.swiglu(np.hstack([g, u])), want, rtol=1e-14, atol=1e-300)


def test_gate_rows_first_then_up_rows():
    """Pairing through the projection: W = [Wg; Wu] with Wg = I and Wu = 2 I
    (K = N/2) makes g = x and u = 2x, so H = 2 x silu(x) -- a swapped or
    shifted pairing would not give this."""
    K = 8
    W = np.zeros((2 * K, K), dtype=np.float32)
    W[:K] = np.eye(K)
    W[K:] = 2.0 * np.eye(K)
    Wb = synth.bf16_from_f32(W)
    x = np.array([[-3.0, -1.0, -0.5, 0.0, 0.25, 1.0, 2.0, 6.0]], dtype=np.float32)
    Xb = synth.bf16_from_f32(x)
    H = oracle.swiglu(oracle.matmul(Xb, Wb))
    xd = x.astype(np.float64)
    assert np.array_equal(H, xd / (1.0 + np.exp(-xd)) * (2.0 * xd))


def test_odd_n_rejected():
    with pytest.raises(ValueError):
        oracle.swiglu(np.zeros((1, 3)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tolerance_accepts_rounded_and_rejects_structural_errors(dtype):
    g, u = _gu(8, 512, 3)
    h = g / (1.0 + np.exp(-g)) * u
    # the device's own error sources: f32 sums, (bf16 operands), f32 evaluation, store
    gp = g.astype(np.float32).astype(np.float64)
    up = u.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        gp = oracle.bf16_bits_to_f64(oracle.round_bf16(gp))
        up = oracle.bf16_bits_to_f64(oracle.round_bf16(up))
    y = (gp / (1.0 + np.exp(-gp)) * up).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        y = oracle.bf16_bits_to_f64(oracle.round_bf16(y))
    assert tolerance.check_swiglu(y, g, u, dtype).ok
    # swapped gate and up, missing activation, shifted pairing: all rejected
    assert not tolerance.check_swiglu(u / (1.0 + np.exp(-u)) * g, g, u, dtype).ok
    assert not tolerance.check_swiglu(g * u, g, u, dtype).ok
    assert not tolerance.check_swiglu(np.roll(h, 1, axis=1), g, u, dtype).ok
