"""Per-tensor dynamic scaling: amax, the exponent bias, and the FP8 cast.

[AMAX] "Proposed method":
  bullet 1 - each tensor's scaling bias comes from that tensor's maximum
             absolute value (FP8-AMAX), for weights, activations, gradients;
  bullet 2 - compute_bias: log2 of (format maximum / tensor amplitude),
             with a configurable margin;
  bullet 3 - the input is scaled before the FP8 cast, and the scaling is
             undone after the matrix multiply.
[FP8LM] "Proposed method", O1, Eq. 3: gradients are multiplied by an
  auto-scaling factor mu (g' = mu * g). Here mu = 2^mu_log2 enters the
  gradient tensor's bias.

Readings (the pages leave these open):
  * the bias is an integer: floor(log2(fmt_max / amax)) - margin + mu_log2,
    the largest shift that keeps amax * 2^bias <= fmt_max when margin = 0;
  * clamped to [-126, 126] so that 2^bias and 2^-bias are normal float32;
  * amax = 0 -> bias 0 with FLAG_ZERO; a NaN or inf in the tensor -> bias 0
    with FLAG_NONFINITE (the cast still runs: NaN -> NaN code, inf -> max);
  * amax is the current tensor's (just-in-time, no history).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from .bf16 import bf16_to_f64
from .formats import Fp8Format, encode

FLAG_NONFINITE = 1
FLAG_ZERO = 2
FLAG_CLAMPED = 4
BIAS_MIN = -126
BIAS_MAX = 126


def amax(bits) -> float:
    """max |t| over a bf16 tensor given as uint16 bit patterns. Returns
    math.nan if any element is NaN, math.inf if any is +-inf (and none is
    NaN), 0.0 for an empty tensor."""
    v = np.abs(bf16_to_f64(np.asarray(bits).reshape(-1)))
    if v.size == 0:
        return 0.0
    if np.isnan(v).any():
        return math.nan
    return float(v.max())


def _floor_log2_ratio(num: Fraction, den: Fraction) -> int:
    """floor(log2(num / den)) for positive rationals, exactly."""
    ratio = num / den
    b = math.floor(math.log2(ratio.numerator) - math.log2(ratio.denominator))
    # correct the float estimate with exact comparisons
    while Fraction(2) ** b > ratio:
        b -= 1
    while Fraction(2) ** (b + 1) <= ratio:
        b += 1
    return b


def compute_bias(amax_value: float, fmt: Fp8Format, margin: int = 0, mu_log2: int = 0):
    """(bias, flags) for one tensor: floor(log2(fmt_max / amax)) - margin +
    mu_log2, clamped to [BIAS_MIN, BIAS_MAX]."""
    if math.isnan(amax_value) or math.isinf(amax_value):
        return 0, FLAG_NONFINITE
    if amax_value == 0.0:
        return 0, FLAG_ZERO
    b = _floor_log2_ratio(Fraction(fmt.max_finite), Fraction(amax_value))
    b = b - margin + mu_log2
    flags = 0
    if b < BIAS_MIN or b > BIAS_MAX:
        flags |= FLAG_CLAMPED
        b = min(max(b, BIAS_MIN), BIAS_MAX)
    return b, flags


def scale_record(bits, fmt: Fp8Format, margin: int = 0, mu_log2: int = 0) -> dict:
    """{amax, bias, scale, scale_inv, flags} for a bf16 tensor."""
    a = amax(bits)
    b, flags = compute_bias(a, fmt, margin, mu_log2)
    return {"amax": a, "bias": b, "scale": 2.0 ** b, "scale_inv": 2.0 ** -b, "flags": flags}


def fixed_record(bias: int) -> dict:
    """FP8-CSCALE [AMAX "Proposed method" bullet 6]: the record of a constant
    scaling bias, set without looking at the tensor (amax 0, no flags)."""
    if not BIAS_MIN <= bias <= BIAS_MAX:
        raise ValueError("bias outside [-126, 126]")
    return {"amax": 0.0, "bias": bias, "scale": 2.0 ** bias, "scale_inv": 2.0 ** -bias, "flags": 0}


def saturated_count(bits, fmt: Fp8Format, bias: int) -> int:
    """Elements that the cast clips: |t| * 2^bias above the format's max
    (an infinity counts, a NaN does not)."""
    x = bf16_to_f64(np.asarray(bits))
    with np.errstate(invalid="ignore", over="ignore"):
        return int(np.count_nonzero(np.abs(np.ldexp(x, bias)) > fmt.max_finite))


def cast(bits, fmt: Fp8Format, bias: int, transposed: bool = True):
    """FP8 codes of t * 2^bias for a bf16 matrix [R, C]: (row-wise [R, C],
    transposed [C, R], or None for it with transposed=False). The product
    is exact in float64."""
    x = bf16_to_f64(bits)
    q = encode(np.ldexp(x, bias), fmt)
    if not transposed:
        return q, None
    return q, np.ascontiguousarray(q.T) if q.ndim == 2 else q
