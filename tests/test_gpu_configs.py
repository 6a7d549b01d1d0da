"""Full-size parity on the five layer workloads, through the C ABI
(fp8_linear_fwd / fp8_linear_bwd: the kernels and launch shapes the
benchmark times, including the forward GEMM's last-wave split where the
workspace enables it).

Per linear, against the oracle on the same seeded inputs:
  * amax, bias, scale and flags of X, W, dY: bit-exact (oracle amax over
    the whole tensor, chunk by chunk);
  * every byte of the row-major FP8 copies x8, w8, dy8: bit-exact (the
    oracle's cast of the whole tensor);
  * Y, dX, dW within 1 bf16 ulp + 1e-4 * sum_r |a_r b_r| of the float64
    oracle on the oracle's FP8 operands:
      - GPT-7B-style and GPT-175B-style layers (the benchmark's workloads):
        every output element, with the workspace exactly as the benchmark
        sets it up (row-major copies only);
      - GPT-125M MLP up, GPT-13B-style and Llama-2-70B-style layers: every
        output element as well, with the transposed copies written too and
        checked equal to the row-major ones transposed (a property at any
        size).
A workload left out of EVERY is checked on the first and the last 256-row
band and a 256-column band of every output (whole rows and whole columns of
tiles, so every tile-row and tile-column index of the tile order is
reached).
"""
import time

import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3, E5M2
import tensor_scaled_fp8_amd as tsf
from tests.fullsize_util import amax_chunked, cast_rows, check_codes, check_gemm, decode
from tests.gpu_util import f32_bits, to_dev_bf16
from workloads import WORKLOADS, linear_inputs

pytestmark = pytest.mark.gpu

EVERY = (1, 2, 3, 4, 5)    # workloads checked on every output element
CASES = [(w, li) for w in sorted(WORKLOADS) for li in range(len(WORKLOADS[w].linears))]


def _check_record(s_dev, bits, fmt, margin, mu):
    a = amax_chunked(bits)
    b, fl = oracle.compute_bias(a, fmt, margin, mu)
    r = tsf.read_scale(s_dev)
    assert f32_bits(r["amax"]) == f32_bits(a)
    assert (r["bias"], r["flags"]) == (b, fl)
    assert r["scale"] == 2.0 ** b
    return b


@pytest.mark.parametrize("wl_idx,li", CASES, ids=[f"{WORKLOADS[w].name}-{WORKLOADS[w].linears[l].name}"
                                                  for w, l in CASES])
def test_full_size_linear(wl_idx, li):
    wl = WORKLOADS[wl_idx]
    L = wl.linears[li]
    every = wl_idx in EVERY
    print(f"\n[full-size] {wl.name} {L.name} M={L.M} K={L.K} N={L.N} every_element={every}", flush=True)
    t0 = time.perf_counter()
    X, W, dY = linear_inputs(wl, li)
    transposed = wl_idx not in (2, 4)
    ws = tsf.LinearWorkspace(L.M, L.K, L.N, transposed=transposed)
    Xd, Wd, dYd = to_dev_bf16(X), to_dev_bf16(W), to_dev_bf16(dY)
    Y = tsf.fp8_linear_fwd(Xd, Wd, ws, wl.margin)
    dX, dW = tsf.fp8_linear_bwd(dYd, ws, wl.margin, wl.mu_log2)
    torch.cuda.synchronize()
    del Xd, Wd, dYd

    bx = _check_record(ws.sx, X, E4M3, wl.margin, 0)
    bw = _check_record(ws.sw, W, E4M3, wl.margin, 0)
    bdy = _check_record(ws.sdy, dY, E5M2, wl.margin, wl.mu_log2)
    x8 = cast_rows(X, E4M3, bx)
    w8 = cast_rows(W, E4M3, bw)
    dy8 = cast_rows(dY, E5M2, bdy)
    del X, W, dY
    check_codes(ws.x8, x8, "x8")
    check_codes(ws.w8, w8, "w8")
    check_codes(ws.dy8, dy8, "dy8")
    if transposed:
        for q, qt in ((ws.x8, ws.x8t), (ws.w8, ws.w8t), (ws.dy8, ws.dy8t)):
            assert torch.equal(qt, q.t()), "transposed copy differs from the row-wise copy"

    xd, wd, dyd = decode(x8, E4M3), decode(w8, E4M3), decode(dy8, E5M2)
    del x8, w8, dy8
    T = 256

    def bands(M, N):
        if every:
            return {}
        g = np.random.Generator(np.random.PCG64(wl_idx * 100 + li))
        last = ((M - 1) // T) * T
        c0 = int(g.integers(0, (N + T - 1) // T)) * T
        return dict(row_bands=[(0, min(T, M)), (last, M)], col_bands=[(c0, min(N, c0 + T))])

    print(f"[full-size] records and FP8 bytes bit-exact ({time.perf_counter() - t0:.1f} s)", flush=True)
    # Y = X W: A = x8 [M, K], B = w8 [K, N]
    n = check_gemm(Y, xd, wd, bx, bw, f"{wl.name}.{L.name} Y", **bands(L.M, L.N))
    print(f"[full-size] Y ok ({n} checked with their sums, {time.perf_counter() - t0:.1f} s)", flush=True)
    # dX = dY W^T: A = dy8 [M, N], B = w8^T [N, K]
    n = check_gemm(dX, dyd, wd.T, bdy, bw, f"{wl.name}.{L.name} dX", **bands(L.M, L.K))
    print(f"[full-size] dX ok ({n} checked with their sums, {time.perf_counter() - t0:.1f} s)", flush=True)
    # dW = X^T dY: A = x8^T [K, M], B = dy8 [M, N]
    n = check_gemm(dW, xd.T, dyd, bx, bdy, f"{wl.name}.{L.name} dW", **bands(L.K, L.N))
    print(f"[full-size] dW ok ({n} checked with their sums, {time.perf_counter() - t0:.1f} s)", flush=True)
