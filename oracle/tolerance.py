"""Acceptance rules for comparing a projection result with the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Rules (written for the weight projection Y = X . W^T, bf16 inputs, f32
accumulation):

* f32-stored Y: every element satisfies ``|y - ref| <= 1e-3 * (|ref| + 1)``,
  ``ref`` the oracle's fp64 value.
* bf16-stored Y: with ``R = bf16_rne(ref)`` and
  ``ulp(R) = 2 ** (max(floor(log2 |R|), -126) - 7)``, an element passes when
  ``|y - R| <= ulp(R)``, or -- near zero, where an f32 accumulation in any order
  legitimately lands several bf16 quanta away from R -- when it meets the f32
  rule above.  The count of elements that needed the second clause is returned
  so that tests can check only tiny-|ref| elements use it.

Why a tolerance and not bit equality: the blog series "On descend d'un cran"
("#002 le meme compilateur sur un GPU", section "Le contrat numerique") states
that correct engines add in different orders and so round differently; any
summation order is a correct result.

Also reported, never gating: the pages' own gate statistic
``max|y - ref| / max|ref|``, which their load-time check bounds by 1/64 ("#004
the same compiler on Apple's chips", section "The night the engine chose
wrong").
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import bf16_bits_to_f64, round_bf16

F32_RTOL = 1e-3


@dataclass
class Report:
    n: int
    n_bad: int
    n_second_clause: int
    worst_excess: float      # max over elements of |err| / allowed  (<= 1 passes)
    gate_ratio: float        # max|y - ref| / max|ref|
    worst_index: int

    @property
    def ok(self) -> bool:
        return self.n_bad == 0

    def __str__(self) -> str:
        return (f"n={self.n} bad={self.n_bad} second_clause={self.n_second_clause} "
                f"worst_excess={self.worst_excess:.3g} (at {self.worst_index}) "
                f"max err {self.gate_ratio:.3e} of max|ref|")


def _gate_ratio(y: np.ndarray, ref: np.ndarray) -> float:
    denom = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(y - ref))) if ref.size else 0.0
    return num / denom if denom > 0 else num


def check_f32(y: np.ndarray, ref: np.ndarray) -> Report:
    y = np.asarray(y, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    if y.shape != ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {ref.shape}")
    allowed = F32_RTOL * (np.abs(ref) + 1.0)
    err = np.abs(y - ref)
    bad = ~(err <= allowed)                      # NaN counts as bad
    excess = np.where(np.isfinite(err), err / allowed, np.inf)
    wi = int(np.argmax(excess)) if y.size else -1
    return Report(n=y.size, n_bad=int(bad.sum()), n_second_clause=0,
                  worst_excess=float(excess[wi]) if y.size else 0.0,
                  gate_ratio=_gate_ratio(y, ref), worst_index=wi)


def bf16_ulp(R: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at R: 2**(max(floor(log2|R|), -126) - 7)."""
    a = np.abs(np.asarray(R, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, e, -126.0)
    e = np.maximum(e, -126.0)
    return np.exp2(e - 7.0)


def check_bf16(y_bits: np.ndarray, ref: np.ndarray) -> Report:
    y_bits = np.asarray(y_bits, dtype=np.uint16).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    if y_bits.shape != ref.shape:
        raise ValueError(f"shape mismatch {y_bits.shape} vs {ref.shape}")
    y = bf16_bits_to_f64(y_bits)
    R = bf16_bits_to_f64(round_bf16(ref))
    ulp = bf16_ulp(R)
    err_R = np.abs(y - R)
    first = err_R <= ulp
    allowed_f32 = F32_RTOL * (np.abs(ref) + 1.0)
    second = np.abs(y - ref) <= allowed_f32
    ok = first | second
    excess = np.minimum(np.where(np.isfinite(err_R), err_R / ulp, np.inf),
                        np.where(np.isfinite(y), np.abs(y - ref) / allowed_f32, np.inf))
    wi = int(np.argmax(excess)) if y.size else -1
    return Report(n=y.size, n_bad=int((~ok).sum()),
                  n_second_clause=int((~first & second).sum()),
                  worst_excess=float(excess[wi]) if y.size else 0.0,
                  gate_ratio=_gate_ratio(y, ref), worst_index=wi)


SILU_LIPSCHITZ = 1.1      # max over x of |d/dx x*sigmoid(x)| = 1.0998...


def check_swiglu(y: np.ndarray, g: np.ndarray, u: np.ndarray, dtype: str) -> Report:
    """A fused SwiGLU output ``y`` [.., N/2] against the oracle's fp64 gate and
    up sums ``g``, ``u`` (``oracle.matmul`` columns [0, N/2) and [N/2, N)).

    Derivation (an allowance per element, from the rules above): the device's
    f32 sums g', u' each meet the projection's f32 rule, |g' - g| <= eg =
    1e-3 (|g| + 1) and likewise eu.  With bf16 storage the epilogue first
    rounds g' and u' to bf16 (relative error <= 2^-9, 2^-8 taken), widening
    eg and eu by 2^-8 of their size.  silu is Lipschitz with constant 1.1, so
    |silu(g')u' - silu(g)u| <= 1.1 eg (|u| + eu) + |silu(g)| eu.  The f32
    evaluation of silu(g')u' adds a few f32 ulps (2^-20 |h| allowed) and a
    bf16 store one more rounding (one bf16 ulp of |h| + the bound).  The
    allowance is of order 1e-3 of the operands: it catches every structural
    mistake (a swapped gate and up, a wrong row pairing, a missing activation
    -- all O(1) changes), while the bit-exactness of the fused result against
    the unfused path is checked separately."""
    y = np.asarray(y, dtype=np.float64).ravel()
    g = np.asarray(g, dtype=np.float64).ravel()
    u = np.asarray(u, dtype=np.float64).ravel()
    if not (y.shape == g.shape == u.shape):
        raise ValueError(f"shape mismatch {y.shape} {g.shape} {u.shape}")
    silu = g / (1.0 + np.exp(-g))
    h = silu * u
    eg = F32_RTOL * (np.abs(g) + 1.0)
    eu = F32_RTOL * (np.abs(u) + 1.0)
    if dtype == "bf16":
        eg = eg + 2.0 ** -8 * (np.abs(g) + eg)
        eu = eu + 2.0 ** -8 * (np.abs(u) + eu)
    allowed = SILU_LIPSCHITZ * eg * (np.abs(u) + eu) + np.abs(silu) * eu + 2.0 ** -20 * np.abs(h)
    if dtype == "bf16":
        allowed = allowed + bf16_ulp(np.abs(h) + allowed)
    err = np.abs(y - h)
    bad = ~(err <= allowed)
    excess = np.where(np.isfinite(err), err / allowed, np.inf)
    wi = int(np.argmax(excess)) if y.size else -1
    return Report(n=y.size, n_bad=int(bad.sum()), n_second_clause=0,
                  worst_excess=float(excess[wi]) if y.size else 0.0,
                  gate_ratio=_gate_ratio(y, h), worst_index=wi)


NORM_REL = 2.0 ** -8    # bf16 rounding of a normalised element (2^-9) plus its f32 scale (taken generously)


def check_norm_projection(y: np.ndarray, ref: np.ndarray, terms: np.ndarray, dtype: str) -> Report:
    """The projection of RMS-normalised rows, ``y`` (f32 values or bf16 bits),
    against the oracle's fp64 ``ref`` (``oracle.rmsnorm_matmul``) and the sums
    of the terms' magnitudes ``terms`` (the same with ``absolute``).

    Derivation: the device multiplies bf16(x r' gamma) by w, where the
    normalised element is rounded to bf16 (relative error <= 2^-9) and r' is
    the f32 scale (relative error well under 2^-12 at any K used here); each
    term is therefore within NORM_REL = 2^-8 of its exact value, and the sum
    within 2^-8 * terms, on top of the projection's own rule (the f32 rule,
    or the bf16 rule for a bf16 Y) for the f32 accumulation and the store."""
    ref = np.asarray(ref, dtype=np.float64).ravel()
    extra = NORM_REL * np.asarray(terms, dtype=np.float64).ravel()
    if dtype == "bf16":
        yv = bf16_bits_to_f64(np.asarray(y, dtype=np.uint16).ravel())
    else:
        yv = np.asarray(y, dtype=np.float64).ravel()
    if yv.shape != ref.shape:
        raise ValueError(f"shape mismatch {yv.shape} vs {ref.shape}")
    a_f32 = F32_RTOL * (np.abs(ref) + 1.0) + extra
    e_f32 = np.abs(yv - ref)
    excess = np.where(np.isfinite(e_f32), e_f32 / a_f32, np.inf)
    if dtype == "bf16":         # within one bf16 ulp of bf16(ref), or the f32 clause
        R = bf16_bits_to_f64(round_bf16(ref))
        a_b = bf16_ulp(R) + extra
        e_b = np.abs(yv - R)
        excess = np.minimum(excess, np.where(np.isfinite(e_b), e_b / a_b, np.inf))
    bad = ~(excess <= 1.0)
    wi = int(np.argmax(excess)) if yv.size else -1
    return Report(n=yv.size, n_bad=int(bad.sum()), n_second_clause=0,
                  worst_excess=float(excess[wi]) if yv.size else 0.0,
                  gate_ratio=_gate_ratio(yv, ref), worst_index=wi)
