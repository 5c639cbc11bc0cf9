"""Exact-arithmetic helpers used to pin the oracle (tests only).

They round an exact rational to f32 or bf16 by bracketing: take the few
representable neighbours of an approximate value and keep the one at the
smallest exact distance, ties to the even bit pattern.  This is a different
method from the oracle's (which scales by the quantum and inspects the
fraction), so a mistake in one does not hide in the other.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

F32_MAX_FINITE = Fraction(np.finfo(np.float32).max.item())


def bf16_value(bits: int) -> Fraction | float:
    """Exact value of a bf16 bit pattern (Fraction), or a float for Inf/NaN."""
    u = np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]
    f = float(u)
    if not np.isfinite(f):
        return f
    return Fraction(f)


def _f32_bits(f: np.float32) -> int:
    return int(np.array([f], dtype=np.float32).view(np.uint32)[0])


def round_to_f32_bits(v: Fraction) -> int:
    """Nearest f32 to the exact value v, ties to even; overflow -> Inf."""
    if v == 0:
        return 0
    approx = np.float32(float(v)) if abs(float(v)) < 3.5e38 else np.float32(np.sign(float(v)) * np.inf)
    cands = set()
    base = approx
    if not np.isfinite(base):
        base = np.float32(np.sign(float(v)) * np.finfo(np.float32).max)
    cands.update([base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(-np.inf))])
    best = None
    for c in cands:
        if not np.isfinite(c):
            # infinity competes as the value 2^128 (IEEE overflow rule)
            cv = Fraction(2) ** 128 * (1 if c > 0 else -1)
        else:
            cv = Fraction(float(c))
        d = abs(cv - v)
        key = (d, _f32_bits(c) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return _f32_bits(best[1])


def round_to_bf16_bits(v: Fraction) -> int:
    """Nearest bf16 to the exact value v, ties to even; overflow -> Inf."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    # approximate pattern: truncate the f32 nearest to a (monotone in a)
    f = np.float32(min(float(a), 3.4e38))
    base = (_f32_bits(f) >> 16) & 0x7FFF
    best = None
    for b in range(max(base - 2, 0), min(base + 3, 0x7F81)):
        if b == 0x7F80:
            cv = Fraction(2) ** 128
        else:
            cv = bf16_value(b)
        d = abs(cv - a)
        key = (d, b & 1)
        if best is None or key < best[0]:
            best = (key, b)
    return sign | best[1]


def exact_dot(x_bits, w_bits) -> Fraction:
    s = Fraction(0)
    for a, b in zip(x_bits, w_bits):
        s += bf16_value(int(a)) * bf16_value(int(b))
    return s
