"""Pins for oracle.gemm / oracle.linear.

Pinned against: exact integer brute force on small shapes (every finite
code class, subnormals and +-max included), one-hot and permutation
operands (whose products reproduce the decoded operand exactly), zero
operands, the symmetry C(A, B) = C(B, A)^T, and the real-valued product of
the unquantised inputs within the quantisation error."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import (E4M3, E5M2, bf16_to_f64, decode_table, f64_to_bf16_rne, gemm_nt,
                    gemm_nt_exact, gemm_nt_rows, linear_fwd_bwd, tolerance, encode)
from workloads import f32_to_bf16_bits


def _finite_codes(fmt):
    t = decode_table(fmt)
    return np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)


def _fraction_to_bf16(fr: Fraction) -> int:
    """Round an exact rational to bf16 (nearest, ties even) without floats."""
    if fr == 0:
        return 0
    sign = 0x8000 if fr < 0 else 0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 7)
    r = a / q
    n = r.numerator // r.denominator
    rem = r - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * q
    f32 = np.array([float(val)], dtype=np.float32)    # exact: val is a bf16 number
    return sign | int(f32.view(np.uint32)[0] >> 16)


@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2)])
def test_gemm_exact_brute_force(fa, fb):
    g = np.random.Generator(np.random.PCG64(21))
    M, N, R = 5, 7, 6                                   # non-square: catches a transposed operand
    A = g.choice(_finite_codes(fa), size=(M, R))
    B = g.choice(_finite_codes(fb), size=(N, R))
    for ba, bb in ((0, 0), (6, 11), (-3, 29)):
        bits, c64, tol = gemm_nt(A, fa, ba, B, fb, bb)
        ex = gemm_nt_exact(A, fa, ba, B, fb, bb)
        for i in range(M):
            for j in range(N):
                e = ex[i][j]
                assert abs(Fraction(c64[i, j]) - e) <= abs(e) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)
                if Fraction(c64[i, j]) == e:
                    assert int(bits[i, j]) == _fraction_to_bf16(e)
        assert np.all(tol > 0)


def test_gemm_one_hot_and_permutation_reproduce_operand():
    g = np.random.Generator(np.random.PCG64(4))
    R = 32
    A = g.choice(_finite_codes(E5M2), size=(9, R))
    one = int(encode(np.array([1.0]), E4M3)[0])
    perm = g.permutation(R)
    B = np.zeros((R, R), np.uint8)
    B[np.arange(R), perm] = one                          # C[:, j] = A[:, perm[j]]
    bits, c64, _ = gemm_nt(A, E5M2, 5, B, E4M3, 2)
    want = decode_table(E5M2)[A][:, perm] * 2.0 ** -7
    assert np.array_equal(c64, want)
    assert np.array_equal(bf16_to_f64(bits), want)       # FP8 values are bf16 values


def test_gemm_zero_and_symmetry():
    g = np.random.Generator(np.random.PCG64(8))
    A = g.choice(_finite_codes(E4M3), size=(12, 48))
    B = g.choice(_finite_codes(E5M2), size=(20, 48))
    Z = np.zeros((20, 48), np.uint8)
    bits, c64, _ = gemm_nt(A, E4M3, 3, Z, E5M2, 1)
    assert not c64.any() and not bits.any()
    _, c_ab, t_ab = gemm_nt(A, E4M3, 3, B, E5M2, 1)
    _, c_ba, _ = gemm_nt(B, E5M2, 1, A, E4M3, 3)
    assert np.all(np.abs(c_ab - c_ba.T) <= 1e-12 * t_ab)
    rows = g.integers(0, 12, 30)
    cols = g.integers(0, 20, 30)
    rb, r64, rt = gemm_nt_rows(A, E4M3, 3, B, E5M2, 1, rows, cols)
    assert np.allclose(r64, c_ab[rows, cols], rtol=1e-13, atol=0)


def test_tolerance_formula_units():
    c = np.array([1.0, -3.0, 0.0])
    s = np.array([10.0, 0.0, 5.0])
    assert np.allclose(tolerance(c, s), [2.0 ** -7 + 1e-3, 2.0 ** -6, 2.0 ** -133 + 5e-4])


def test_linear_approximates_real_product():
    """The three GEMMs approximate X W, dY W^T and X^T dY of the unquantised
    bf16 inputs: relative error of a few percent at FP8 precision, and the
    outputs have the right shapes (a dropped or inverted scale would be off
    by a power of two; a transposed operand by much more)."""
    g = np.random.Generator(np.random.PCG64(2))
    M, K, N = 48, 80, 64
    X = f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    W = f32_to_bf16_bits((0.02 * g.standard_normal((K, N))).astype(np.float32))
    dY = f32_to_bf16_bits((1e-5 * g.standard_normal((M, N))).astype(np.float32))
    out = linear_fwd_bwd(X, W, dY, margin=0)
    x, w, dy = bf16_to_f64(X), bf16_to_f64(W), bf16_to_f64(dY)
    for key, ref in (("Y", x @ w), ("dX", dy @ w.T), ("dW", x.T @ dy)):
        got = out[key][1]
        assert got.shape == ref.shape
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel < 0.08, (key, rel)
    assert out["sx"]["bias"] == compute_bias_ref(X, 448.0)
    assert out["sdy"]["bias"] == compute_bias_ref(dY, 57344.0)


def compute_bias_ref(bits, mx):
    import math
    a = float(np.abs(bf16_to_f64(bits)).max())
    return math.floor(math.log2(mx / a))
