"""FP8 number formats: the 256-code decode table and the saturating
round-to-nearest-even encoder.

[AMAX] "Proposed method", bullet 4: weights and activations use the E4
format, gradients the E5 format. The pages name the formats only; the
encodings below are the OCP 8-bit formats (a reading), whose largest finite
values are 448 (E4M3) and 57344 (E5M2):

  E4M3: sign | 4 exponent bits (bias 7) | 3 mantissa bits. No infinities;
        S.1111.111 is NaN, so the top binade stops at 1.75 * 2^8 = 448.
  E5M2: sign | 5 exponent bits (bias 15) | 2 mantissa bits. S.11111.00 is
        +-inf, S.11111.{01,10,11} are NaN; max 1.75 * 2^15 = 57344.
  Exponent field 0 holds subnormals (m * 2^(1 - bias - mbits)) and +-0.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Fp8Format:
    name: str
    exp_bits: int
    man_bits: int
    exp_bias: int
    max_finite: float
    ieee_specials: bool   # True: all-ones exponent is inf/NaN (E5M2); False: only S.1111.111 is NaN

    @property
    def emin(self) -> int:            # exponent of the smallest normal
        return 1 - self.exp_bias

    @property
    def max_code(self) -> int:        # positive code of max_finite
        return 0x7E if not self.ieee_specials else 0x7B

    @property
    def nan_code(self) -> int:        # positive quiet-NaN code emitted by the encoder
        return 0x7F


E4M3 = Fp8Format("e4m3", 4, 3, 7, 448.0, False)
E5M2 = Fp8Format("e5m2", 5, 2, 15, 57344.0, True)
FORMATS = {"e4m3": E4M3, "e5m2": E5M2, 0: E4M3, 1: E5M2}


def decode_code(code: int, fmt: Fp8Format) -> float:
    """Value of one 8-bit code, straight from the field definitions."""
    s = (code >> 7) & 1
    e = (code >> fmt.man_bits) & ((1 << fmt.exp_bits) - 1)
    m = code & ((1 << fmt.man_bits) - 1)
    sign = -1.0 if s else 1.0
    e_all = (1 << fmt.exp_bits) - 1
    if fmt.ieee_specials and e == e_all:
        return sign * math.inf if m == 0 else math.nan
    if (not fmt.ieee_specials) and e == e_all and m == (1 << fmt.man_bits) - 1:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** (fmt.emin - fmt.man_bits)
    return sign * (1.0 + m / (1 << fmt.man_bits)) * 2.0 ** (e - fmt.exp_bias)


def decode_table(fmt: Fp8Format) -> np.ndarray:
    """The 256-entry decode table, float64, indexed by the code."""
    return np.array([decode_code(c, fmt) for c in range(256)], dtype=np.float64)


def encode(values, fmt: Fp8Format) -> np.ndarray:
    """Encode float64 values to FP8 codes: round to nearest, ties to the
    even code, saturating every magnitude above max_finite (inf included)
    to +-max_finite; NaN -> 0x7F with the sign bit; subnormals kept; the
    sign of values that round to zero is kept (-> 0x80).

    The steps: take the binade e = max(floor(log2|v|), emin), the spacing
    q = 2^(e - mbits) in it, and r = |v| / q rounded half-to-even (exact,
    q is a power of two). r < 2^mbits only in the subnormal binade; r equal
    to 2^(mbits+1) carries into the next binade.
    """
    v = np.asarray(values, dtype=np.float64)
    shape = v.shape
    v = v.reshape(-1)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.uint8)

    nan = np.isnan(v)
    sat = (~nan) & (a > fmt.max_finite)
    fin = (~nan) & (~sat) & (a > 0)

    mb = fmt.man_bits
    af = a[fin]
    _, ex = np.frexp(af)                   # af = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, fmt.emin)
    q = np.ldexp(1.0, e - mb)
    r = np.rint(af / q).astype(np.int64)   # np.rint: half to even
    carry = r == (1 << (mb + 1))
    e = np.where(carry, e + 1, e)
    r = np.where(carry, 1 << mb, r)
    normal = r >= (1 << mb)
    field_e = np.where(normal, e + fmt.exp_bias, 0)
    field_m = np.where(normal, r - (1 << mb), r)
    code = (field_e << mb) | field_m
    # rounding up to a value above max (cannot happen once a <= max) guarded anyway
    code = np.minimum(code, fmt.max_code)
    out[fin] = code.astype(np.uint8)
    out[sat] = fmt.max_code
    out[nan] = fmt.nan_code
    out |= sign
    return out.reshape(shape)
