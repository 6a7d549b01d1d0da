"""FP8 weight gradient with the amax fused into the wgrad epilogue
(fp8_wgrad_fp8), through the C ABI.

[FP8-LM reading note, "Proposed method", O1, Eq. 3: FP8 gradients with the
auto-scaling factor mu; Perez et al. review, "Proposed method" bullet 4: E5
for gradients]. dW (bf16) is the a6 GEMM and is checked against the float64
oracle within the GEMM tolerance. The integers that follow from it — amax,
bias, flags, every E5M2 byte and the clipped-element count — are checked bit
for bit against the oracle applied to the kernel's own dW (both sides decide
them from the same bf16 values). The call must also equal the unfused
sequence (wgrad GEMM, then fp8_quantize of dW) byte for byte.
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


def _operands(M, K, N, seed, dy_sigma=1e-5, x_sigma=1.0):
    g = np.random.Generator(np.random.PCG64(seed))
    xb = oracle.f64_to_bf16_rne(g.standard_normal((M, K)) * x_sigma)
    dyb = oracle.f64_to_bf16_rne(g.standard_normal((M, N)) * dy_sigma)
    return xb, dyb


def _fp8_operands(xb, dyb, margin, mu):
    M, K = xb.shape
    N = dyb.shape[1]
    sx, sdy = tsf.new_scale(1)[0], tsf.new_scale(1)[0]
    _, x8t = tsf.fp8_quantize(to_dev_bf16(xb), "e4m3", sx, margin, 0, rowwise=False)
    _, dy8t = tsf.fp8_quantize(to_dev_bf16(dyb), "e5m2", sdy, margin, mu, rowwise=False)
    return x8t, sx, dy8t, sdy


def _check_chain(dW, dw8, dw8t, s_dw, margin, mu):
    bits = bf16_bits(dW)
    rec = oracle.scale_record(bits, E5M2, margin, mu)
    r = tsf.read_scale(s_dw)
    assert f32_bits(r["amax"]) == f32_bits(rec["amax"])
    assert (r["bias"], r["flags"]) == (rec["bias"], rec["flags"])
    assert r["scale"] == rec["scale"] and r["scale_inv"] == rec["scale_inv"]
    q, qt = oracle.cast(bits, E5M2, rec["bias"])
    assert np.array_equal(u8(dw8), q)
    if dw8t is not None:
        assert np.array_equal(u8(dw8t), qt)
    assert r["sat_count"] == oracle.saturated_count(bits, E5M2, rec["bias"])
    return rec


def _check_dw_vs_oracle(dW, xb, dyb, bx, bdy):
    qa, _ = oracle.cast(np.ascontiguousarray(xb.T), E4M3, bx)
    qb, _ = oracle.cast(np.ascontiguousarray(dyb.T), E5M2, bdy)
    want, _, tol = oracle.gemm_nt(qa, E4M3, bx, qb, E5M2, bdy)
    err = np.abs(oracle.bf16_to_f64(bf16_bits(dW)) - oracle.bf16_to_f64(want))
    bad = ~(err <= tol)
    assert not bad.any(), (int(bad.sum()), float((err / tol).max()))


@pytest.mark.parametrize("M,K,N,margin,mu", [(400, 272, 528, 0, 0), (256, 256, 256, 1, 0), (512, 768, 3072, 0, 2),
                                             (784, 2064, 272, 0, -1), (16, 16, 16, 0, 0), (128, 528, 1040, 2, 3)])
def test_wgrad_fp8_matches_oracle_and_unfused(M, K, N, margin, mu):
    xb, dyb = _operands(M, K, N, M + 3 * K + 7 * N)
    x8t, sx, dy8t, sdy = _fp8_operands(xb, dyb, margin, mu)
    dW, dw8, dw8t, s_dw = tsf.fp8_wgrad_fp8(x8t, sx, dy8t, sdy, margin, mu, transposed=True)
    torch.cuda.synchronize()
    bx, bdy = tsf.read_scale(sx)["bias"], tsf.read_scale(sdy)["bias"]
    _check_dw_vs_oracle(dW, xb, dyb, bx, bdy)
    _check_chain(dW, dw8, dw8t, s_dw, margin, mu)
    # unfused: the wgrad GEMM, then fp8_quantize of dW
    dW2 = tsf.fp8_gemm_nt(x8t, "e4m3", sx, dy8t, "e5m2", sdy)
    s2 = tsf.new_scale(1)[0]
    q2, qt2 = tsf.fp8_quantize(dW2, "e5m2", s2, margin, mu)
    torch.cuda.synchronize()
    assert torch.equal(dW.view(torch.int16), dW2.view(torch.int16))
    assert torch.equal(dw8, q2) and torch.equal(dw8t, qt2)
    r1, r2 = tsf.read_scale(s_dw), tsf.read_scale(s2)
    assert all(r1[k] == r2[k] for k in ("bias", "flags", "scale")) and f32_bits(r1["amax"]) == f32_bits(r2["amax"])


def test_mu_above_margin_clips_and_counts():
    """With mu > 1 the largest gradients clip at the E5M2 max; the count
    equals the oracle's, and it is zero at mu = 1."""
    M, K, N = 512, 384, 640
    xb, dyb = _operands(M, K, N, 11)
    x8t, sx, dy8t, sdy = _fp8_operands(xb, dyb, 0, 0)
    counts = []
    for mu in (0, 1, 3, 6):
        dW, dw8, _, s_dw = tsf.fp8_wgrad_fp8(x8t, sx, dy8t, sdy, 0, mu)
        torch.cuda.synchronize()
        _check_chain(dW, dw8, None, s_dw, 0, mu)
        counts.append(tsf.read_scale(s_dw)["sat_count"])
    assert counts[0] == 0 and counts[1] > 0 and counts[1] < counts[2] < counts[3]


def test_zero_and_empty_gradients():
    M, K, N = 64, 96, 160
    xb, _ = _operands(M, K, N, 5)
    dyb = np.zeros((M, N), np.uint16)
    x8t, sx, dy8t, sdy = _fp8_operands(xb, dyb, 0, 0)
    s_dw = tsf.new_scale(1)[0]
    for _ in range(2):                      # the second call reuses the record
        dW, dw8, _, s_dw = tsf.fp8_wgrad_fp8(x8t, sx, dy8t, sdy, s_dw=s_dw)
        torch.cuda.synchronize()
        r = tsf.read_scale(s_dw)
        assert (r["amax"], r["bias"], r["flags"], r["sat_count"]) == (0.0, 0, tsf.FLAG_ZERO, 0)
        assert not torch.any(dw8)
    # K = 0: nothing to compute, the record still publishes
    e8 = torch.zeros((0, 64), dtype=torch.uint8, device="cuda")
    d8 = torch.zeros((16, 64), dtype=torch.uint8, device="cuda")
    dW, dw8, _, s_e = tsf.fp8_wgrad_fp8(e8, sx, d8, sdy)
    torch.cuda.synchronize()
    assert dW.shape == (0, 16) and tsf.read_scale(s_e)["flags"] == tsf.FLAG_ZERO


def test_record_reuse_with_shrinking_gradients():
    """Generation tagging: each call's amax is its own, also when it is
    smaller than the previous call's."""
    M, K, N = 256, 272, 528
    s_dw = tsf.new_scale(1)[0]
    for i, sigma in enumerate((1e-3, 1e-6, 1e-4, 1e-9)):
        xb, dyb = _operands(M, K, N, 40 + i, dy_sigma=sigma)
        x8t, sx, dy8t, sdy = _fp8_operands(xb, dyb, 0, 0)
        dW, dw8, _, _ = tsf.fp8_wgrad_fp8(x8t, sx, dy8t, sdy, s_dw=s_dw)
        torch.cuda.synchronize()
        _check_chain(dW, dw8, None, s_dw, 0, 0)


@pytest.mark.parametrize("M,K,N,margin,mu", [(400, 272, 528, 0, 0), (784, 2064, 272, 0, -1), (16, 16, 16, 0, 0),
                                             (128, 528, 1040, 2, 3)])
def test_wgrad_fp8_row_major_operands(M, K, N, margin, mu):
    """The row-major FP8 copies X [M,K] and dY [M,N], read reduction-major,
    against the transposed copies read row-wise: the two run different tile
    bodies of the GEMM (rounding FP32 partial sums at different k
    boundaries), so each dW is held to the GEMM tolerance against the
    oracle, and each call's record, E5M2 codes and clipped count are checked
    bit for bit against the oracle applied to its own dW."""
    xb, dyb = _operands(M, K, N, M + 5 * K + 3 * N)
    x8t, sx, dy8t, sdy = _fp8_operands(xb, dyb, margin, mu)
    x8, _ = tsf.fp8_quantize(to_dev_bf16(xb), "e4m3", tsf.new_scale(1)[0], margin, 0, transposed=False)
    dy8, _ = tsf.fp8_quantize(to_dev_bf16(dyb), "e5m2", tsf.new_scale(1)[0], margin, mu, transposed=False)
    a = tsf.fp8_wgrad_fp8(x8t, sx, dy8t, sdy, margin, mu, transposed=True)
    b = tsf.fp8_wgrad_fp8(x8, sx, dy8, sdy, margin, mu, transposed=True, x_layout="cols", dy_layout="cols")
    torch.cuda.synchronize()
    bx, bdy = tsf.read_scale(sx)["bias"], tsf.read_scale(sdy)["bias"]
    for dW, dw8, dw8t, s_dw in (a, b):
        _check_dw_vs_oracle(dW, xb, dyb, bx, bdy)
        _check_chain(dW, dw8, dw8t, s_dw, margin, mu)


@pytest.mark.parametrize("M,K,N", [(400, 272, 528), (784, 2064, 272)])
@pytest.mark.parametrize("x_layout,dy_layout", [("rows", "cols"), ("cols", "rows")])
def test_wgrad_fp8_mixed_layouts(M, K, N, x_layout, dy_layout):
    """One operand as its transposed copy (read row-wise), the other as the
    row-major copy (read reduction-major): dW within the GEMM tolerance of
    the oracle, and the record, E5M2 codes and clipped count bit-exact
    against the oracle applied to the kernel's own dW. (rows, cols) is the
    fused-amax layout that runs on the 32 x 32 x 64 tile body although its
    A is row-layout."""
    margin, mu = 0, 1
    xb, dyb = _operands(M, K, N, 7 * M + K + N + (x_layout == "rows"))
    x8t, sx, dy8t, sdy = _fp8_operands(xb, dyb, margin, mu)
    x8, _ = tsf.fp8_quantize(to_dev_bf16(xb), "e4m3", tsf.new_scale(1)[0], margin, 0, transposed=False)
    dy8, _ = tsf.fp8_quantize(to_dev_bf16(dyb), "e5m2", tsf.new_scale(1)[0], margin, mu, transposed=False)
    xo = x8t if x_layout == "rows" else x8
    dyo = dy8t if dy_layout == "rows" else dy8
    dW, dw8, dw8t, s_dw = tsf.fp8_wgrad_fp8(xo, sx, dyo, sdy, margin, mu, transposed=True, x_layout=x_layout,
                                            dy_layout=dy_layout)
    torch.cuda.synchronize()
    bx, bdy = tsf.read_scale(sx)["bias"], tsf.read_scale(sdy)["bias"]
    _check_dw_vs_oracle(dW, xb, dyb, bx, bdy)
    _check_chain(dW, dw8, dw8t, s_dw, margin, mu)


def test_wgrad_fp8_full_size_gpt7b_up():
    """Full size (dW 4096 x 16384 from 4096 tokens), from the training
    step's row-major FP8 copies: record and every E5M2 byte bit-exact vs the
    oracle on the kernel's dW, and identical to the unfused sequence."""
    wl = WORKLOADS[2]
    li = [l.name for l in wl.linears].index("up")
    L = wl.linears[li]
    X, W, dY = linear_inputs(wl, li)
    ws = tsf.LinearWorkspace(L.M, L.K, L.N)
    tsf.fp8_linear_fwd(to_dev_bf16(X), to_dev_bf16(W), ws)
    tsf.fp8_linear_bwd(to_dev_bf16(dY), ws, need_dx=False, need_dw=False)
    dW, dw8, _, s_dw = tsf.fp8_wgrad_fp8(ws.x8, ws.sx, ws.dy8, ws.sdy, wl.margin, 0, x_layout="cols",
                                         dy_layout="cols")
    dW2 = tsf.fp8_gemm(ws.x8, "e4m3", ws.sx, ws.dy8, "e5m2", ws.sdy, a_layout="cols", b_layout="cols")
    s2 = tsf.new_scale(1)[0]
    q2, _ = tsf.fp8_quantize(dW2, "e5m2", s2, transposed=False)
    torch.cuda.synchronize()
    assert torch.equal(dW.view(torch.int16), dW2.view(torch.int16))
    assert torch.equal(dw8, q2)
    bits = bf16_bits(dW)
    rec = oracle.scale_record(bits, E5M2, wl.margin, 0)
    r = tsf.read_scale(s_dw)
    assert f32_bits(r["amax"]) == f32_bits(rec["amax"]) and (r["bias"], r["flags"]) == (rec["bias"], rec["flags"])
    assert r["sat_count"] == oracle.saturated_count(bits, E5M2, rec["bias"])
    rows = np.random.Generator(np.random.PCG64(7)).choice(L.K, size=64, replace=False)
    assert np.array_equal(u8(dw8[torch.from_numpy(rows).cuda()]), oracle.cast(bits[rows], E5M2, rec["bias"])[0])
