"""Pins for the CPU oracle: each test fixes it against something other than itself.

The pages of "On descend d'un cran" print no numeric input or output of any
projection, so the oracle is pinned by brute force, closed forms, special cases
and invariants.  Each group names the mistake it is meant to catch.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import tolerance
from tests import exact
import synth


def _rand_bf16(rng, shape, emin=-8, emax=8):
    """Random bf16 bit patterns with exponent in [emin, emax], random sign and
    7-bit mantissa.  In that range every double accumulation below is exact."""
    e = rng.integers(emin, emax + 1, size=shape)
    mant = rng.integers(0, 128, size=shape)
    sign = rng.integers(0, 2, size=shape)
    return ((sign << 15) | ((e + 127) << 7) | mant).astype(np.uint16)


# ---------------------------------------------------------------- P1 brute force
@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_tiny_exact_then_rounded(seed):
    """All M, N, K <= 5: the oracle's fp64 sum equals the exact rational sum, and
    its f32 / bf16 roundings equal an independent bracketing rounding of it.
    Catches a dropped term, a wrong index, a wrong widening or a wrong rounding."""
    rng = np.random.default_rng(seed)
    for M in range(1, 6):
        for N in range(1, 6):
            for K in range(1, 6):
                X = _rand_bf16(rng, (M, K))
                W = _rand_bf16(rng, (N, K))
                Y = oracle.matmul(X, W)
                Y32 = oracle.round_f32(Y)
                Y16 = oracle.round_bf16(Y)
                for m in range(M):
                    for n in range(N):
                        ex = exact.exact_dot(X[m], W[n])
                        assert Fraction(Y[m, n]) == ex, (M, N, K, m, n)
                        assert int(Y32[m:m + 1, n:n + 1].view(np.uint32)[0, 0]) == \
                            exact.round_to_f32_bits(ex)
                        assert int(Y16[m, n]) == exact.round_to_bf16_bits(ex)


def test_bruteforce_wide_range_within_bound():
    """With bf16 inputs spanning a wide exponent range the fp64 sum may round;
    it must stay within K * 2^-53 * sum|x*w| of the exact sum."""
    rng = np.random.default_rng(11)
    for _ in range(40):
        M, N, K = (int(v) for v in rng.integers(1, 6, size=3))
        X = _rand_bf16(rng, (M, K), -60, 60)
        W = _rand_bf16(rng, (N, K), -60, 60)
        Y = oracle.matmul(X, W)
        for m in range(M):
            for n in range(N):
                ex = exact.exact_dot(X[m], W[n])
                mag = sum(abs(exact.bf16_value(int(a)) * exact.bf16_value(int(b)))
                          for a, b in zip(X[m], W[n]))
                assert abs(Fraction(Y[m, n]) - ex) <= K * Fraction(1, 2 ** 53) * mag


# ---------------------------------------------------------------- P2 integer probes
@pytest.mark.parametrize("M,N,K", [(3, 17, 1024), (16, 64, 17408), (5, 151, 2560)])
def test_integer_probe_exact(M, N, K):
    """Integer-valued bf16 in [-4, 4]: every partial sum is an integer below 2^24,
    so the result is known exactly (numpy int64 product as the independent
    closed form), and the f32 result equals it bit for bit."""
    X = synth.int_bf16(1, (M, K))
    W = synth.int_bf16(2, (N, K))
    Xi = oracle.bf16_bits_to_f64(X).astype(np.int64)
    Wi = oracle.bf16_bits_to_f64(W).astype(np.int64)
    ref = Xi @ Wi.T
    Y = oracle.matmul(X, W)
    assert np.array_equal(Y, ref.astype(np.float64))
    assert np.array_equal(oracle.round_f32(Y), ref.astype(np.float32))
    # bf16: RNE of the exact integer, checked by bracketing on a sample
    Y16 = oracle.round_bf16(Y)
    flat = ref.ravel()
    for i in np.random.default_rng(0).choice(flat.size, size=min(200, flat.size), replace=False):
        assert int(Y16.ravel()[i]) == exact.round_to_bf16_bits(Fraction(int(flat[i])))


# ---------------------------------------------------------------- P3 special cases
def test_identity_weights():
    rng = np.random.default_rng(3)
    K = 96
    X = synth.bf16_from_f32(rng.standard_normal((7, K)).astype(np.float32))
    eye = synth.bf16_from_f32(np.eye(K, dtype=np.float32))
    Y = oracle.matmul(X, eye)
    assert np.array_equal(Y, oracle.bf16_bits_to_f64(X))


def test_permutation_weights():
    """W = P (a permutation): Y[:, n] = X[:, perm[n]].  Catches a transposed W."""
    rng = np.random.default_rng(4)
    K = 64
    perm = rng.permutation(K)
    P = np.zeros((K, K), dtype=np.float32)
    P[np.arange(K), perm] = 1.0
    X = synth.bf16_from_f32(rng.standard_normal((5, K)).astype(np.float32))
    Y = oracle.matmul(X, synth.bf16_from_f32(P))
    assert np.array_equal(Y, oracle.bf16_bits_to_f64(X)[:, perm])


def test_one_hot_rows_select_columns_of_w():
    """X row m = e_j: Y[m, :] = W[:, j].  With N != K this also pins which
    operand is transposed."""
    rng = np.random.default_rng(5)
    N, K = 37, 23
    W = synth.bf16_from_f32(rng.standard_normal((N, K)).astype(np.float32))
    js = [0, 5, 22]
    X = np.zeros((len(js), K), dtype=np.float32)
    for m, j in enumerate(js):
        X[m, j] = 1.0
    Y = oracle.matmul(synth.bf16_from_f32(X), W)
    for m, j in enumerate(js):
        assert np.array_equal(Y[m], oracle.bf16_bits_to_f64(W[:, j]))


def test_k_equals_one_is_outer_product():
    rng = np.random.default_rng(6)
    X = synth.bf16_from_f32(rng.standard_normal((4, 1)).astype(np.float32))
    W = synth.bf16_from_f32(rng.standard_normal((9, 1)).astype(np.float32))
    Y = oracle.matmul(X, W)
    assert np.array_equal(Y, np.outer(oracle.bf16_bits_to_f64(X[:, 0]),
                                      oracle.bf16_bits_to_f64(W[:, 0])))


def test_empty_shapes():
    X = np.zeros((0, 8), dtype=np.uint16)
    W = np.zeros((3, 8), dtype=np.uint16)
    assert oracle.matmul(X, W).shape == (0, 3)
    assert oracle.matmul(np.zeros((2, 8), np.uint16), np.zeros((0, 8), np.uint16)).shape == (2, 0)


def test_rows_entry_matches_full():
    rng = np.random.default_rng(7)
    X = _rand_bf16(rng, (20, 40), -20, 20)
    W = _rand_bf16(rng, (33, 40), -20, 20)
    full = oracle.matmul(X, W)
    rows = [19, 0, 7, 7]
    assert np.array_equal(oracle.matmul_rows(X, rows, W), full[rows])


# ---------------------------------------------------------------- P4 / P5 invariants
@pytest.mark.parametrize("a,b", [(1, 1), (2, -1), (-0.5, 2), (0.5, 0.5), (-2, -0.5)])
def test_linearity_in_x(a, b):
    """oracle(a X1 + b X2) = a oracle(X1) + b oracle(X2) exactly, with every input
    exactly representable and every accumulation exact."""
    rng = np.random.default_rng(8)
    K, M, N = 48, 6, 11
    X1 = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    X2 = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    W = _rand_bf16(rng, (N, K), -8, 8)
    Xc = np.float32(a) * X1 + np.float32(b) * X2
    Y = oracle.matmul(synth.bf16_from_f32(Xc), W)
    Y1 = oracle.matmul(synth.bf16_from_f32(X1), W)
    Y2 = oracle.matmul(synth.bf16_from_f32(X2), W)
    assert np.array_equal(Y, a * Y1 + b * Y2)


@pytest.mark.parametrize("shift", [-20, -3, 1, 9])
def test_power_of_two_scaling(shift):
    rng = np.random.default_rng(9)
    X = _rand_bf16(rng, (4, 64), -8, 8)
    W = _rand_bf16(rng, (10, 64), -8, 8)
    Xs = synth.bf16_from_f32(oracle.bf16_bits_to_f64(X).astype(np.float32) * np.float32(2.0 ** shift))
    assert np.array_equal(oracle.matmul(Xs, W), oracle.matmul(X, W) * 2.0 ** shift)


# ---------------------------------------------------------------- P6 library cross-check
@pytest.mark.parametrize("M,N,K", [(1, 300, 1024), (9, 77, 3072), (16, 33, 17408)])
def test_against_numpy_float64(M, N, K):
    X = synth.normal_bf16(99, 0, (M, K), 1.0)
    W = synth.normal_bf16(99, 1, (N, K), 0.02, outlier_frac=0.01)
    Xd = oracle.bf16_bits_to_f64(X)
    Wd = oracle.bf16_bits_to_f64(W)
    ref = Xd @ Wd.T
    mag = np.abs(Xd) @ np.abs(Wd).T
    Y = oracle.matmul(X, W)
    assert np.all(np.abs(Y - ref) <= 2 * K * 2.0 ** -53 * mag + 1e-300)


# ---------------------------------------------------------------- rounding pins
def test_bf16_roundtrip_all_patterns():
    """Every non-NaN bf16 value converts back to its own bit pattern (+-0,
    subnormals, max finite, +-Inf included)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    back = oracle.round_bf16(vals)
    finite_or_inf = ~np.isnan(vals)
    assert np.array_equal(back[finite_or_inf], bits[finite_or_inf])
    assert np.all((back[~finite_or_inf] & 0x7FC0) == 0x7FC0)


def test_bf16_midpoints_tie_to_even():
    """The exact midpoint between consecutive positive bf16 values goes to the
    even pattern; a hair above goes up, a hair below goes down.  The midpoint
    above the largest finite value overflows to +Inf."""
    lo = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    hi = (lo.astype(np.uint32) + 1).astype(np.uint16)
    vlo = oracle.bf16_bits_to_f64(lo)
    vhi = np.where(hi == 0x7F80, 2.0 ** 128, oracle.bf16_bits_to_f64(hi))
    mid = (vlo + vhi) / 2           # exact in double
    got = oracle.round_bf16(mid)
    want = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(got, want)
    up = oracle.round_bf16(np.nextafter(mid, np.inf))
    dn = oracle.round_bf16(np.nextafter(mid, -np.inf))
    assert np.array_equal(up, hi) and np.array_equal(dn, lo)
    # negative side mirrors the positive side
    assert np.array_equal(oracle.round_bf16(-mid), want | 0x8000)


def test_bf16_special_values():
    assert oracle.f64_to_bf16(0.0) == 0x0000
    assert oracle.f64_to_bf16(-0.0) == 0x8000
    assert oracle.f64_to_bf16(float("inf")) == 0x7F80
    assert oracle.f64_to_bf16(float("-inf")) == 0xFF80
    assert oracle.f64_to_bf16(float("nan")) & 0x7FC0 == 0x7FC0
    assert oracle.f64_to_bf16(1e300) == 0x7F80
    assert oracle.f64_to_bf16(2.0 ** -134) == 0x0000        # half the least subnormal: tie to 0
    assert oracle.f64_to_bf16(3 * 2.0 ** -135) == 0x0001    # 0.75 quantum -> 1 quantum
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80    # tie -> even (1.0)
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.f64_to_bf16(-1.0 - 2.0 ** -8 - 2.0 ** -40) == 0xBF81


def test_f32_to_bf16_matches_library_cast():
    """f32 -> bf16 through the oracle equals torch's RNE cast on 2^22 random and
    all boundary-adjacent f32 patterns (NaN excluded)."""
    rng = np.random.default_rng(12)
    pats = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    edges = []
    for hi in range(0, 0x10000, 1):
        base = hi << 16
        edges += [base + 0x7FFF, base + 0x8000, base + 0x8001]
    pats = np.concatenate([pats, np.array(edges, dtype=np.uint64).astype(np.uint32)])
    f = pats.view(np.float32)
    keep = ~np.isnan(f)
    f = f[keep]
    mine = oracle.round_f32_to_bf16(f)
    lib = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, lib)


# ---------------------------------------------------------------- tolerance rule
def test_tolerance_rules():
    ref = np.array([0.0, 1.0, -1000.0, 1e-5, 3.0])
    ok = ref + np.array([9e-4, 1.9e-3, 0.9, -5e-4, 3.9e-3])
    bad = ref + np.array([1.1e-3, 2.1e-3, 1.01, 1.1e-3, 4.1e-3])
    assert tolerance.check_f32(ok, ref).ok
    assert tolerance.check_f32(bad, ref).n_bad == 5
    assert tolerance.check_f32(np.array([np.nan]), np.array([0.0])).n_bad == 1
    # bf16 rule: 1 ulp of the rounded reference
    ref2 = np.array([1.0, 100.0, -3.0])
    R = oracle.round_bf16(ref2)
    one_up = (R.astype(np.int32) + 1).astype(np.uint16)
    two_up = (R.astype(np.int32) + 2).astype(np.uint16)
    assert tolerance.check_bf16(one_up, ref2).ok
    rep = tolerance.check_bf16(two_up, ref2)
    assert rep.n_bad == 3
    # near zero the second clause rescues a few-ulp gap
    tiny = np.array([1.3e-5])
    y = oracle.round_bf16(tiny + 4e-7)
    rep = tolerance.check_bf16(y, tiny)
    assert rep.ok and rep.n_second_clause == 1
    assert tolerance.bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert tolerance.bf16_ulp(np.array([0.0]))[0] == 2.0 ** -133
