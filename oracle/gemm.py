"""The three FP8 GEMMs of the linear, as one NT contraction.

[AMAX] "Proposed method", bullet 3: the matrix multiply runs on the FP8
operands and the per-tensor scaling is undone afterwards. With the NT form

    C[i, j] = 2^-(bias_a + bias_b) * sum_r dec(A)[i, r] * dec(B)[j, r]

(both operands row-major, reduction dimension contiguous) the forward is
Y = X W (A = x8 [M,K], B = w8t [N,K]), the data gradient dX = dY W^T
(A = dy8 [M,N], B = w8 [K,N]) and the weight gradient dW = X^T dY
(A = x8t [K,M], B = dy8t [N,M]). The output is rounded once to bf16,
nearest-even (a reading: the pages leave the output type open).

The reference sum is taken in float64 (a BLAS dgemm as a library step);
`gemm_nt_exact` computes it with Python integers for small pins.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .bf16 import bf16_ulp, f64_to_bf16_rne
from .formats import Fp8Format, decode_table

TOL_REL = 1e-4


def _decode(codes, fmt: Fp8Format) -> np.ndarray:
    return decode_table(fmt)[np.asarray(codes, dtype=np.uint8)]


def gemm_nt(a_codes, fmt_a: Fp8Format, bias_a: int, b_codes, fmt_b: Fp8Format, bias_b: int,
            with_tolerance: bool = True):
    """Returns (C bf16 bits [M,N], C float64 before rounding, tolerance
    [M,N] or None)."""
    A = _decode(a_codes, fmt_a)
    B = _decode(b_codes, fmt_b)
    s = 2.0 ** (-(bias_a + bias_b))
    c64 = (A @ B.T) * s
    bits = f64_to_bf16_rne(c64)
    tol = None
    if with_tolerance:
        abs_sum = (np.abs(A) @ np.abs(B).T) * s
        tol = tolerance(c64, abs_sum)
    return bits, c64, tol


def gemm_nt_rows(a_codes, fmt_a, bias_a, b_codes, fmt_b, bias_b, rows, cols):
    """Selected outputs C[rows[t], cols[t]] only (for sampled checks at
    full size). Returns (bits, c64, tol), each of shape [len(rows)]."""
    ta, tb = decode_table(fmt_a), decode_table(fmt_b)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    A = ta[np.asarray(a_codes)[rows]]
    B = tb[np.asarray(b_codes)[cols]]
    s = 2.0 ** (-(bias_a + bias_b))
    c64 = np.einsum("tr,tr->t", A, B) * s
    abs_sum = np.einsum("tr,tr->t", np.abs(A), np.abs(B)) * s
    return f64_to_bf16_rne(c64), c64, tolerance(c64, abs_sum)


def tolerance(c_ref, abs_prod_sum):
    """Allowed |C_device - C_ref|: one bf16 ulp of the reference plus
    1e-4 * sum_r |a_r * b_r| (same units as the output)."""
    return bf16_ulp(c_ref) + TOL_REL * np.asarray(abs_prod_sum, dtype=np.float64)


def gemm_nt_exact(a_codes, fmt_a: Fp8Format, bias_a: int, b_codes, fmt_b: Fp8Format, bias_b: int):
    """Exact rational C (before rounding) by brute force: every FP8 value is
    an integer times 2^(emin - mbits), so products and sums are integer
    arithmetic. Small shapes only. Returns a list of lists of Fraction."""
    ta, tb = decode_table(fmt_a), decode_table(fmt_b)
    ua = 2 ** (fmt_a.exp_bias - 1 + fmt_a.man_bits)     # 1 / (smallest subnormal)
    ub = 2 ** (fmt_b.exp_bias - 1 + fmt_b.man_bits)
    A = [[int(ta[c] * ua) for c in row] for row in np.asarray(a_codes)]
    B = [[int(tb[c] * ub) for c in row] for row in np.asarray(b_codes)]
    den = Fraction(ua * ub) * Fraction(2) ** (bias_a + bias_b)
    out = []
    for ra in A:
        out.append([Fraction(sum(x * y for x, y in zip(ra, rb))) / den for rb in B])
    return out
