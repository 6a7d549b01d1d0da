"""fp8_gemm_ws: the forward GEMM with its last partial wave split into
reduction halves, through the C ABI.

[Perez et al. review, "Proposed method", bullet 3: the matmul runs on the
scaled FP8 operands and the scaling is undone after it.] A split tile is
the FP32 sum of two half-reduction partials (half 0 + half 1), then the
same dequantising bf16 epilogue: a different accumulation order from the
unsplit kernel, so the bar is the GEMM tolerance against the float64
oracle (|C - C_oracle| <= 1 bf16 ulp + 1e-4 * 2^-(ba+bb) * sum_r |a_r b_r|),
plus determinism (two calls give the same bits), bit-identity with
fp8_gemm where nothing splits (shape not eligible, workspace too small)
and, at full size, that the split happened (some tiles differ from the
unsplit result) on exactly the tail's tiles' worth of outputs at most."""
import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3
import tensor_scaled_fp8_amd as tsf
from tests.gpu_util import bf16_bits, scale_record, to_dev_u8

pytestmark = pytest.mark.gpu


def _codes(shape, sigma, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return oracle.encode(g.standard_normal(shape) * sigma, E4M3)


def _run(A, B, la, lb, ws=None, out=None, split="tail"):
    a = to_dev_u8(np.ascontiguousarray(A.T) if la == "cols" else A)
    b = to_dev_u8(np.ascontiguousarray(B.T) if lb == "cols" else B)
    return tsf.fp8_gemm(a, "e4m3", scale_record(6), b, "e4m3", scale_record(11), out=out, a_layout=la, b_layout=lb,
                        workspace=ws, split=split)


def _check_oracle(C, A, B):
    bits, _, tol = oracle.gemm_nt(A, E4M3, 6, B, E4M3, 11)
    err = np.abs(oracle.bf16_to_f64(bf16_bits(C)) - oracle.bf16_to_f64(bits))
    assert not np.any(~(err <= tol)), float(np.max(err / tol))


@pytest.mark.parametrize("M,N,R", [(784, 272, 2048), (1040, 528, 1024), (16, 16, 1024), (256, 256, 4096),
                                   (272, 1040, 1536)])
@pytest.mark.parametrize("la,lb", [("rows", "rows"), ("rows", "cols"), ("cols", "rows"), ("cols", "cols")])
def test_split_matches_oracle_and_is_deterministic(M, N, R, la, lb):
    A, B = _codes((M, R), 6.0, M + 3 * N + R), _codes((N, R), 40.0, M + 5 * N + R)
    nb = tsf.gemm_workspace_bytes("e4m3", "e4m3", M, N, R, "tail")
    assert nb > 0   # every tile of these shapes is in a last wave under half full
    assert tsf.gemm_workspace_bytes("e4m3", "e4m3", M, N, R, "auto") == 0   # too short to pay
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    C1 = _run(A, B, la, lb, ws)
    C2 = _run(A, B, la, lb, ws)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    _check_oracle(C1, A, B)


def test_no_split_paths_equal_fp8_gemm():
    """Ineligible shape (R not a multiple of 256), a too small workspace, no
    workspace, split "never" or "auto" below its reduction threshold, and a
    backward format pair all give fp8_gemm's bits."""
    A, B = _codes((272, 1040), 6.0, 1), _codes((528, 1040), 40.0, 2)
    ref = _run(A, B, "rows", "cols")
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    assert tsf.gemm_workspace_bytes("e4m3", "e4m3", 272, 528, 1040, "tail") == 0
    out = _run(A, B, "rows", "cols", ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    A2, B2 = _codes((272, 2048), 6.0, 9), _codes((528, 2048), 40.0, 10)
    ref2 = _run(A2, B2, "rows", "cols")
    for mode in ("never", "auto"):
        out = _run(A2, B2, "rows", "cols", ws, split=mode)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref2.view(torch.int16)), mode
    A, B = _codes((272, 1024), 6.0, 3), _codes((528, 1024), 40.0, 4)
    ref = _run(A, B, "rows", "cols")
    small = torch.empty(tsf.gemm_workspace_bytes("e4m3", "e4m3", 272, 528, 1024, "tail") - 16, dtype=torch.uint8,
                        device="cuda")
    out = _run(A, B, "rows", "cols", small)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    dy = to_dev_u8(oracle.encode(np.random.Generator(np.random.PCG64(5)).standard_normal((272, 1024)) * 1e3,
                                 oracle.E5M2))
    w = to_dev_u8(B)
    r1 = tsf.fp8_gemm(dy, "e5m2", scale_record(23), w, "e4m3", scale_record(11))
    r2 = tsf.fp8_gemm(dy, "e5m2", scale_record(23), w, "e4m3", scale_record(11), workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(r1.view(torch.int16), r2.view(torch.int16))


def test_linear_forward_with_scratch_matches_oracle():
    """fp8_linear_fwd with the workspace's scratch (a shape whose forward
    splits under the automatic rule: R = K = 16384)."""
    from workloads import draw_normal_bf16
    from tests.gpu_util import to_dev_bf16
    M, K, N = 512, 16384, 768
    xb, wb = draw_normal_bf16(11, (M, K), 1.0), draw_normal_bf16(12, (K, N), 0.02)
    ws = tsf.LinearWorkspace(M, K, N)
    assert ws.scratch is not None and ws.scratch.numel() == tsf.load().fp8_linear_scratch_bytes(M, K, N)
    Y = tsf.fp8_linear_fwd(to_dev_bf16(xb), to_dev_bf16(wb), ws)
    torch.cuda.synchronize()
    bx = oracle.scale_record(xb, E4M3)["bias"]
    bw = oracle.scale_record(wb, E4M3)["bias"]
    qx = oracle.cast(xb, E4M3, bx)[0]
    qw = oracle.cast(wb, E4M3, bw)[0]
    bits, _, tol = oracle.gemm_nt(qx, E4M3, bx, np.ascontiguousarray(qw.T), E4M3, bw)
    err = np.abs(oracle.bf16_to_f64(bf16_bits(Y)) - oracle.bf16_to_f64(bits))
    assert not np.any(~(err <= tol)), float(np.max(err / tol))


def test_full_size_gpt175b_proj_forward():
    """2048 x 12288 x 12288 (the GPT-175B-style proj forward): 384 tiles,
    a 128-tile tail on 256 CUs. Against the unsplit kernel: the split
    happened (some tiles differ) and only within at most ntail tiles; the
    last 16 rows (a row of tiles, tail tiles among them) against the
    oracle."""
    M = 2048
    N = R = 12288
    nb = tsf.gemm_workspace_bytes("e4m3", "e4m3", M, N, R, "tail")
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = (M // 256) * (N // 256)
    if nb == 0:
        pytest.skip(f"{tiles} tiles leave no split tail on {ncu} CUs")
    ntail = nb // (2 * 65536 * 4)
    assert ntail == tiles % ncu
    g = torch.Generator(device="cuda")
    g.manual_seed(175)
    a = (torch.randn((M, R), device="cuda", generator=g) * 6).to(torch.float8_e4m3fn).view(torch.uint8)
    w = (torch.randn((R, N), device="cuda", generator=g) * 40).to(torch.float8_e4m3fn).view(torch.uint8)
    sa, sb = scale_record(6), scale_record(11)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ref = tsf.fp8_gemm(a, "e4m3", sa, w, "e4m3", sb, b_layout="cols")
    C = tsf.fp8_gemm(a, "e4m3", sa, w, "e4m3", sb, b_layout="cols", workspace=ws, split="tail")
    torch.cuda.synchronize()
    diff = (C.view(torch.int16) != ref.view(torch.int16)).view(M // 256, 256, N // 256, 256)
    tiles_diff = int(diff.any(dim=3).any(dim=1).sum())
    assert 0 < tiles_diff <= ntail, tiles_diff
    a_h, w_h = a.cpu().numpy(), w.cpu().numpy()
    rows = slice(M - 16, M)
    bits, _, tol = oracle.gemm_nt(a_h[rows], E4M3, 6, np.ascontiguousarray(w_h.T), E4M3, 11)
    got = oracle.bf16_to_f64(bf16_bits(C[rows]))
    err = np.abs(got - oracle.bf16_to_f64(bits))
    assert not np.any(~(err <= tol)), float(np.max(err / tol))
