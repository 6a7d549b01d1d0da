"""Helpers for full-size parity: the oracle's own steps applied to whole
workload tensors, chunk by chunk on a thread pool (numpy releases the GIL
in its element-wise kernels, and the float64 products run in BLAS), so a
complete comparison of every FP8 byte and every GEMM output element fits in
the host memory and the time of one test.

No method arithmetic here beyond calling the oracle: the casts are
oracle.cast on row chunks, the GEMM sums are float64 products of the
oracle's decode-table values, and the comparison applies oracle.tolerance.
One shortcut keeps the element-wise pass cheap and is exact with respect
to that tolerance: where |C_gpu - c| <= ulp_bf16(c) / 2 for the float64
sum c, the bound |C_gpu - bf16(c)| <= ulp_bf16(c) already holds (the
rounding of c moves it by at most half its ulp), so such elements pass the
tolerance whatever sum_r |a_r b_r| is; every other element is checked in
full, with its sum_r |a_r b_r| computed from its row and column.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from tests.gpu_util import bf16_bits, u8

_POOL = ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))
_CHUNK = 1 << 22          # elements per task


def _row_chunks(rows: int, cols: int):
    step = max(1, _CHUNK // max(cols, 1))
    return [(r, min(rows, r + step)) for r in range(0, rows, step)]


def cast_rows(bits: np.ndarray, fmt, bias: int) -> np.ndarray:
    """oracle.cast of a whole [R, C] bf16 tensor (row-wise codes), in row chunks."""
    R, C = bits.shape
    out = np.empty((R, C), np.uint8)

    def one(rc):
        r0, r1 = rc
        out[r0:r1] = oracle.cast(bits[r0:r1], fmt, bias, transposed=False)[0]
    list(_POOL.map(one, _row_chunks(R, C)))
    return out


def decode(codes: np.ndarray, fmt) -> np.ndarray:
    """float64 values of FP8 codes through the oracle's decode table."""
    tab = oracle.decode_table(fmt)
    flat = codes.reshape(-1)
    out = np.empty(flat.shape, np.float64)

    def one(rc):
        r0, r1 = rc
        out[r0:r1] = tab[flat[r0:r1]]
    list(_POOL.map(one, _row_chunks(flat.size, 1)))
    return out.reshape(codes.shape)


def amax_chunked(bits, chunk=1 << 24) -> float:
    flat = bits.reshape(-1)
    vals = list(_POOL.map(lambda i: oracle.amax(flat[i:i + chunk]), range(0, flat.size, chunk))) or [0.0]
    if any(np.isnan(v) for v in vals):
        return float("nan")
    return max(vals)


def check_codes(dev: torch.Tensor, want: np.ndarray, name: str) -> None:
    """Every byte of a device FP8 copy equals the oracle's."""
    got = u8(dev)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{name}: {len(bad)} FP8 bytes differ from the oracle, first "
                             f"{[(tuple(i), int(got[tuple(i)]), int(want[tuple(i)])) for i in bad[:6]]}")


def _exact_abs_sum(a_rows, b_mat, ii, jj) -> np.ndarray:
    """sum_r |a[i, r] b[r, j]| in float64 for the listed elements (gathers
    of 256 rows and columns at a time)."""
    out = np.empty(len(ii))
    for t0 in range(0, len(ii), 256):
        t1 = min(len(ii), t0 + 256)
        out[t0:t1] = np.einsum("tr,rt->t", np.abs(a_rows[ii[t0:t1]]), np.abs(b_mat[:, jj[t0:t1]]))
    return out


class _Abs32:
    """|x| in float32, computed once on first use (shared by the bands)."""

    def __init__(self, x):
        self.x, self.v = x, None

    def get(self):
        if self.v is None:
            self.v = np.empty(self.x.shape, np.float32)
            rows = self.x.shape[0]

            def one(rc):
                r0, r1 = rc
                self.v[r0:r1] = np.abs(self.x[r0:r1])
            list(_POOL.map(one, _row_chunks(rows, self.x.shape[1])))
        return self.v


def _check_band(got_bits: np.ndarray, c64: np.ndarray, a_rows: np.ndarray, b_mat: np.ndarray, scale: float,
                where: str, a_abs32=None, b_abs32=None) -> int:
    """Band of outputs against the float64 sums c64 (see the module note).
    a_rows [rows, R] and b_mat [R, cols] are the decoded operands of the band.
    Elements outside the half-ulp shortcut get their sum_r |a_r b_r|: from a
    float64 gather when they are few; when they are many, first from one
    float32 product of the band's absolute values, lowered by its rounding
    bound (float32 holds every product of two FP8 values exactly, and a
    sum of R positive terms carries a relative error below gamma_R =
    R u / (1 - R u), u = 2^-24), so that it never exceeds the exact sum;
    an element that fails with that lower bound is checked with its exact
    float64 sum. Returns how many elements left the shortcut."""
    rows = c64.shape[0]
    slow = []

    def one(rc):
        r0, r1 = rc
        g = oracle.bf16_to_f64(got_bits[r0:r1])
        c = c64[r0:r1]
        with np.errstate(invalid="ignore"):
            ok = np.abs(g - c) <= 0.5 * oracle.bf16_ulp(c)
        idx = np.argwhere(~ok)
        if idx.size:
            slow.append(idx + np.array([r0, 0]))
    list(_POOL.map(one, _row_chunks(rows, c64.shape[1])))
    if not slow:
        return 0
    idx = np.concatenate(slow)
    ii, jj = idx[:, 0], idx[:, 1]
    c = c64[ii, jj]
    want = oracle.bf16_to_f64(oracle.f64_to_bf16_rne(c))
    err = np.abs(oracle.bf16_to_f64(got_bits[ii, jj]) - want)
    if len(idx) <= 4096:
        tol = oracle.tolerance(c, _exact_abs_sum(a_rows, b_mat, ii, jj) * scale)
        bad = ~(err <= tol)
    else:
        R = a_rows.shape[1]
        gamma = R * 2.0 ** -24 / (1 - R * 2.0 ** -24)
        aa = a_abs32() if a_abs32 else np.abs(a_rows).astype(np.float32)
        bb = b_abs32() if b_abs32 else np.abs(b_mat).astype(np.float32)
        s32 = aa @ bb
        lower = s32[ii, jj].astype(np.float64) * (1 - gamma) * scale
        bad = ~(err <= oracle.tolerance(c, lower))
        if bad.any():       # settle those with the exact sum
            bi = np.flatnonzero(bad)
            tol = oracle.tolerance(c[bi], _exact_abs_sum(a_rows, b_mat, ii[bi], jj[bi]) * scale)
            bad[bi] = ~(err[bi] <= tol)
    assert not bad.any(), (where, int(bad.sum()), [(int(i), int(j)) for i, j in idx[bad][:6]],
                           float(np.nanmax(err[bad])))
    return int(len(idx))


def check_gemm(out_dev: torch.Tensor, a_dec: np.ndarray, b_mat: np.ndarray, bias_a: int, bias_b: int,
               where: str, row_bands=None, col_bands=None, band: int = 1024) -> int:
    """out[i, j] = bf16(2^-(ba+bb) * sum_r a_dec[i, r] b_mat[r, j]) within the
    oracle tolerance: every element (row_bands = col_bands = None), or the
    listed row bands (whole rows of the output) and column bands (whole
    columns), each (start, stop). a_dec [M, R] and b_mat [R, N] may be
    transposed views. Returns the count of elements checked in full."""
    M, N = out_dev.shape
    scale = 2.0 ** (-(bias_a + bias_b))
    slow = 0
    if row_bands is None and col_bands is None:
        row_bands = [(r, min(M, r + band)) for r in range(0, M, band)]
    b_abs = _Abs32(b_mat)
    for r0, r1 in row_bands or []:
        a = a_dec[r0:r1]
        c64 = (a @ b_mat) * scale
        got = bf16_bits(out_dev[r0:r1])
        slow += _check_band(got, c64, a, b_mat, scale, f"{where} rows {r0}:{r1}", b_abs32=b_abs.get)
    a_abs = _Abs32(a_dec)
    for c0, c1 in col_bands or []:
        b = np.ascontiguousarray(b_mat[:, c0:c1])
        c64 = (a_dec @ b) * scale
        got = bf16_bits(out_dev[:, c0:c1])
        slow += _check_band(got, c64, a_dec, b, scale, f"{where} cols {c0}:{c1}", a_abs32=a_abs.get)
    return slow
