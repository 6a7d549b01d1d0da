"""bf16 <-> float64 helpers: exact widening, and a single
round-to-nearest-even narrowing from float64 (no intermediate float32)."""
from __future__ import annotations

import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_BF16_OVERFLOW = (2.0 - 2.0 ** -8) * 2.0 ** 127   # >= this rounds to inf


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_rne(values) -> np.ndarray:
    """float64 -> bf16 bits, one rounding, to nearest, ties to even.
    Normal binades keep 8 significant bits; below 2^-126 the spacing is
    2^-133. Magnitudes from (2 - 2^-8) * 2^127 up become inf."""
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex.astype(np.int64) - 1, -126)
    q = np.ldexp(1.0, e - 7)
    r = np.rint(np.where(np.isfinite(a), a, 0.0) / q) * q   # exact in float64
    r = np.where(a >= _BF16_OVERFLOW, np.inf, r)
    r = np.where(np.isinf(a), np.inf, r)
    r = np.copysign(r, v)
    r = np.where(np.isnan(v), np.nan, r)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # exact: r is a bf16 value
    return bits


def bf16_ulp(values) -> np.ndarray:
    """Spacing of bf16 numbers at |v|: 2^(floor(log2|v|) - 7) for
    |v| >= 2^-126, else 2^-133 (also for v = 0)."""
    a = np.abs(np.asarray(values, dtype=np.float64))
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = ex.astype(np.int64) - 1
    ulp = np.ldexp(1.0, e - 7)
    return np.where(a >= 2.0 ** -126, ulp, 2.0 ** -133)
