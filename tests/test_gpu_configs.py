"""Full-size parity on the five layer workloads, through the C ABI
(fp8_linear_fwd / fp8_linear_bwd, the same kernels and launch shapes the
benchmark times).

At these sizes the oracle checks, per linear:
  * amax, bias, scale and flags of X, W, dY: bit-exact (oracle amax over the
    whole tensor, taken chunk by chunk);
  * FP8 bytes: bit-exact on 48 sampled rows of each row-wise copy and 48
    sampled rows of each transposed copy (oracle cast of those rows or
    columns), plus, on the device, transposed copy == row-wise copy
    transposed for the whole tensor (a property at any size);
  * Y, dX, dW: 192 sampled elements each, plus two whole 256 x 256 output
    tiles (one interior tile and the last, bottom-right one, i.e. complete
    kernel tiles), within 1 bf16 ulp + 1e-4 * sum_r |a_r b_r| of the float64
    oracle on the oracle's own FP8 operands.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3, E5M2
import tensor_scaled_fp8_amd as tsf
from tests.gpu_util import bf16_bits, f32_bits, to_dev_bf16, u8
from workloads import WORKLOADS, linear_inputs

pytestmark = pytest.mark.gpu

CASES = [(w, li) for w in sorted(WORKLOADS) for li in range(len(WORKLOADS[w].linears))]
N_ROWS = 48
N_OUT = 192


def _amax_chunked(bits, chunk=1 << 24):
    flat = bits.reshape(-1)
    vals = [oracle.amax(flat[i:i + chunk]) for i in range(0, flat.size, chunk)] or [0.0]
    if any(np.isnan(v) for v in vals):
        return float("nan")
    return max(vals)


def _check_record(s_dev, bits, fmt, margin, mu):
    a = _amax_chunked(bits)
    b, fl = oracle.compute_bias(a, fmt, margin, mu)
    r = tsf.read_scale(s_dev)
    assert f32_bits(r["amax"]) == f32_bits(a)
    assert (r["bias"], r["flags"]) == (b, fl)
    assert r["scale"] == 2.0 ** b
    return b


def _check_cast(bits, fmt, bias, q_dev, qt_dev, g):
    R, Cc = bits.shape
    rows = g.choice(R, size=min(N_ROWS, R), replace=False)
    cols = g.choice(Cc, size=min(N_ROWS, Cc), replace=False)
    want_rows, _ = oracle.cast(bits[rows], fmt, bias)
    want_cols, _ = oracle.cast(np.ascontiguousarray(bits[:, cols].T), fmt, bias)
    assert np.array_equal(u8(q_dev[torch.from_numpy(rows).cuda()]), want_rows)
    assert np.array_equal(u8(qt_dev[torch.from_numpy(cols).cuda()]), want_cols)
    assert torch.equal(qt_dev, q_dev.t()), "transposed copy differs from the row-wise copy"


def _check_gemm(out_dev, a_bits, fa, ba, b_bits_t, fb, bb, g):
    """out[i, j] = sum_r A[i, r] B[j, r]; A rows from a_bits (bf16 [M, R]),
    B rows from b_bits_t (bf16 [N, R]), both cast by the oracle."""
    M, N = out_dev.shape
    ii = g.integers(0, M, N_OUT)
    jj = g.integers(0, N, N_OUT)
    ua, inv_a = np.unique(ii, return_inverse=True)
    ub, inv_b = np.unique(jj, return_inverse=True)
    qa, _ = oracle.cast(a_bits(ua), fa, ba)
    qb, _ = oracle.cast(b_bits_t(ub), fb, bb)
    bits, c64, tol = oracle.gemm_nt_rows(qa, fa, ba, qb, fb, bb, inv_a, inv_b)
    got = bf16_bits(out_dev[torch.from_numpy(ii).cuda(), torch.from_numpy(jj).cuda()])
    err = np.abs(oracle.bf16_to_f64(got) - oracle.bf16_to_f64(bits))
    bad = ~(err <= tol)
    assert not bad.any(), (int(bad.sum()), float((err / tol).max()))
    # whole output tiles: one interior tile and the last one
    T = 256
    tiles = [(int(g.integers(0, max(1, M // T))) * T, int(g.integers(0, max(1, N // T))) * T),
             (max(0, M - T), max(0, N - T))]
    for r0, c0 in tiles:
        rows = np.arange(r0, min(M, r0 + T))
        cols = np.arange(c0, min(N, c0 + T))
        qa, _ = oracle.cast(a_bits(rows), fa, ba)
        qb, _ = oracle.cast(b_bits_t(cols), fb, bb)
        bits, c64, tol = oracle.gemm_nt(qa, fa, ba, qb, fb, bb)
        got = bf16_bits(out_dev[r0:r0 + len(rows), c0:c0 + len(cols)])
        err = np.abs(oracle.bf16_to_f64(got) - oracle.bf16_to_f64(bits))
        bad = ~(err <= tol)
        assert not bad.any(), ("tile", r0, c0, int(bad.sum()), float((err / tol).max()))


@pytest.mark.parametrize("wl_idx,li", CASES, ids=[f"{WORKLOADS[w].name}-{WORKLOADS[w].linears[l].name}"
                                                  for w, l in CASES])
def test_full_size_linear(wl_idx, li):
    wl = WORKLOADS[wl_idx]
    L = wl.linears[li]
    X, W, dY = linear_inputs(wl, li)
    ws = tsf.LinearWorkspace(L.M, L.K, L.N, transposed=True)
    Xd, Wd, dYd = to_dev_bf16(X), to_dev_bf16(W), to_dev_bf16(dY)
    Y = tsf.fp8_linear_fwd(Xd, Wd, ws, wl.margin)
    dX, dW = tsf.fp8_linear_bwd(dYd, ws, wl.margin, wl.mu_log2)
    torch.cuda.synchronize()
    del Xd, Wd, dYd
    g = np.random.Generator(np.random.PCG64(wl_idx * 100 + li))

    bx = _check_record(ws.sx, X, E4M3, wl.margin, 0)
    bw = _check_record(ws.sw, W, E4M3, wl.margin, 0)
    bdy = _check_record(ws.sdy, dY, E5M2, wl.margin, wl.mu_log2)
    _check_cast(X, E4M3, bx, ws.x8, ws.x8t, g)
    _check_cast(W, E4M3, bw, ws.w8, ws.w8t, g)
    _check_cast(dY, E5M2, bdy, ws.dy8, ws.dy8t, g)

    # Y = X W: A rows = X rows, B rows = W columns
    _check_gemm(Y, lambda r: X[r], E4M3, bx, lambda c: np.ascontiguousarray(W[:, c].T), E4M3, bw, g)
    # dX = dY W^T: A rows = dY rows, B rows = W rows
    _check_gemm(dX, lambda r: dY[r], E5M2, bdy, lambda c: W[c], E4M3, bw, g)
    # dW = X^T dY: A rows = X columns, B rows = dY columns
    _check_gemm(dW, lambda r: np.ascontiguousarray(X[:, r].T), E4M3, bx,
                lambda c: np.ascontiguousarray(dY[:, c].T), E5M2, bdy, g)
