"""fp8_gemm with reduction-major operands (FP8_OPERAND_COLS), through the C ABI.

[Perez et al. review, "Proposed method", bullet 3: the matmul runs on the
scaled FP8 operands.] A reduction-major operand is the row-major FP8 copy
of a tensor read transposed (A [R, M], B [R, N]), so the forward and the
weight-gradient GEMMs need no transposed FP8 copies. The kernel has two
bodies of its tile: the 16 x 16 x 128 MFMA one wherever A has one row per
output index, the 32 x 32 x 64 one for a reduction-major A. Within a body
the MFMAs see the same k-bytes per lane whatever B's layout, so (rows,
rows) and (rows, cols) must agree bit for bit, as must (cols, rows) and
(cols, cols); the two bodies round their FP32 partial sums at different k
boundaries, so every layout is held to the GEMM tolerance against the
float64 oracle. Shapes cover partial tiles in M and N (chunks past the
edge read the last valid chunk), partial last stages in R (zero-filled
k-rows), the smallest sizes and every format pair."""
import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3, E5M2
import tensor_scaled_fp8_amd as tsf
from tests.gpu_util import bf16_bits, scale_record, to_dev_u8

pytestmark = pytest.mark.gpu
FMT = {0: E4M3, 1: E5M2}
NAME = {0: "e4m3", 1: "e5m2"}
LAYOUTS = [("rows", "cols"), ("cols", "rows"), ("cols", "cols")]
BODY = {("rows", "rows"): "k128", ("rows", "cols"): "k128", ("cols", "rows"): "k64", ("cols", "cols"): "k64"}


def _operands(M, N, R, fa, fb, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    A = oracle.encode(g.standard_normal((M, R)) * 40, FMT[fa])
    B = oracle.encode(g.standard_normal((N, R)) * 40, FMT[fb])
    return A, B


def _run(A, fa, ba, B, fb, bb, la, lb):
    a = to_dev_u8(np.ascontiguousarray(A.T) if la == "cols" else A)
    b = to_dev_u8(np.ascontiguousarray(B.T) if lb == "cols" else B)
    return tsf.fp8_gemm(a, NAME[fa], scale_record(ba), b, NAME[fb], scale_record(bb), a_layout=la, b_layout=lb)


@pytest.mark.parametrize("M,N,R", [(272, 528, 400), (256, 256, 128), (16, 16, 16), (784, 272, 2064),
                                   (16, 1040, 528), (512, 768, 144), (48, 32, 1040)])
@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_layouts_bit_identical_and_oracle(M, N, R, fa, fb):
    A, B = _operands(M, N, R, fa, fb, M + 3 * N + 7 * R + 11 * fa + 13 * fb)
    bits, _, tol = oracle.gemm_nt(A, FMT[fa], 6, B, FMT[fb], 11)
    first = {}
    for la, lb in [("rows", "rows")] + LAYOUTS:
        out = _run(A, fa, 6, B, fb, 11, la, lb)
        torch.cuda.synchronize()
        err = np.abs(oracle.bf16_to_f64(bf16_bits(out)) - oracle.bf16_to_f64(bits))
        assert not np.any(~(err <= tol)), (la, lb, float(np.max(err / tol)))
        ref = first.setdefault(BODY[(la, lb)], out)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (la, lb)


def test_layouts_one_hot_exact():
    """B = permutation of 1.0 codes, read reduction-major: C reproduces
    columns of A exactly (pins the k pairing of the transposing reads)."""
    g = np.random.Generator(np.random.PCG64(78))
    codes = np.array([c for c in range(256) if np.isfinite(oracle.decode_table(E4M3)[c])], np.uint8)
    for M, R in ((32, 64), (288, 320), (16, 16)):
        A = g.choice(codes, size=(M, R))
        one = int(oracle.encode(np.array([1.0]), E4M3)[0])
        perm = g.permutation(R)
        B = np.zeros((R, R), np.uint8)
        B[np.arange(R), perm] = one
        want, _, _ = oracle.gemm_nt(A, E4M3, 2, B, E4M3, -1)
        for la, lb in LAYOUTS:
            out = _run(A, 0, 2, B, 0, -1, la, lb)
            torch.cuda.synchronize()
            assert np.array_equal(bf16_bits(out), want), (M, R, la, lb)


def _differing_within_tolerance(out, ref, a_rows, b_rows, fa, fb, ba, bb, limit):
    """Elements where out and ref differ: few (at most limit), and out is
    within the GEMM tolerance of the float64 oracle at each of them (the
    exact sum of its row of A and row of B, decoded on the host)."""
    idx = (out.view(torch.int16) != ref.view(torch.int16)).nonzero().cpu().numpy()
    assert len(idx) <= limit, len(idx)
    if len(idx) == 0:
        return 0
    ii, jj = idx[:, 0], idx[:, 1]
    a = oracle.decode_table(fa)[a_rows[torch.from_numpy(ii).cuda()].cpu().numpy()]
    b = oracle.decode_table(fb)[b_rows[torch.from_numpy(jj).cuda()].cpu().numpy()]
    scale = 2.0 ** -(ba + bb)
    c = np.einsum("tr,tr->t", a, b) * scale
    abs_sum = np.einsum("tr,tr->t", np.abs(a), np.abs(b)) * scale
    want = oracle.bf16_to_f64(oracle.f64_to_bf16_rne(c))
    got = oracle.bf16_to_f64(bf16_bits(out)[ii, jj])
    tol = oracle.tolerance(c, abs_sum)
    assert np.all(np.abs(got - want) <= tol), float(np.max(np.abs(got - want) / tol))
    return len(idx)


def test_layouts_full_size_gpt7b_shapes():
    """The step's reduction-major GEMMs at full size. The forward of up
    (4096 x 16384 x 4096, B = w8 reduction-major) equals the row-layout GEMM
    on the transposed copy bit for bit (same tile body). The weight
    gradient of down (16384 x 4096 x 4096, both operands reduction-major)
    equals (cols, rows) bit for bit (same body, B read both ways); where it
    differs from the row-layout GEMM (the other body: rare last-bit
    roundings, at most one in 10^4 elements here), each such element is
    within the GEMM tolerance of the float64 oracle."""
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    s_a, s_b = scale_record(6), scale_record(11)
    for (M, N, R), (la, lb) in (((4096, 16384, 4096), ("rows", "cols")), ((16384, 4096, 4096), ("cols", "cols"))):
        a_rows = torch.randint(0, 0x78, (M, R), dtype=torch.uint8, device="cuda", generator=g)
        b_rows = torch.randint(0, 0x78, (N, R), dtype=torch.uint8, device="cuda", generator=g)
        a = a_rows.t().contiguous() if la == "cols" else a_rows
        b = b_rows.t().contiguous() if lb == "cols" else b_rows
        ref = tsf.fp8_gemm_nt(a_rows, "e4m3", s_a, b_rows, "e5m2", s_b)
        out = tsf.fp8_gemm(a, "e4m3", s_a, b, "e5m2", s_b, a_layout=la, b_layout=lb)
        torch.cuda.synchronize()
        if la == "rows":
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (M, N, R, la, lb)
            continue
        same_body = tsf.fp8_gemm(a, "e4m3", s_a, b_rows, "e5m2", s_b, a_layout="cols", b_layout="rows")
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), same_body.view(torch.int16)), (M, N, R)
        _differing_within_tolerance(out, ref, a_rows, b_rows, E4M3, E5M2, 6, 11, M * N // 10000)


def test_layouts_operand_of_2gib():
    """A 2 GiB B operand (N x R = 2^31 bytes, the top bit of the 32-bit
    offsets in use) in both layouts: the results are identical, and sampled
    output columns equal the oracle's within tolerance."""
    M, N, R = 256, 65536, 32768
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    a = torch.randint(0, 0x78, (M, R), dtype=torch.uint8, device="cuda", generator=g)
    b_rows = torch.randint(0, 0x78, (N, R), dtype=torch.uint8, device="cuda", generator=g)
    s_a, s_b = scale_record(3), scale_record(4)
    ref = tsf.fp8_gemm(a, "e4m3", s_a, b_rows, "e4m3", s_b)
    cols = torch.from_numpy(np.random.Generator(np.random.PCG64(12)).choice(N, size=6, replace=False)).cuda()
    cols = torch.cat([cols, torch.tensor([0, N - 1], device="cuda")])
    b_sample = b_rows[cols].cpu().numpy()
    b_t = b_rows.t().contiguous()
    del b_rows
    out = tsf.fp8_gemm(a, "e4m3", s_a, b_t, "e4m3", s_b, b_layout="cols")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    bits, _, tol = oracle.gemm_nt(a.cpu().numpy(), E4M3, 3, b_sample, E4M3, 4)
    got = oracle.bf16_to_f64(bf16_bits(out[:, cols]))
    assert np.all(np.abs(got - oracle.bf16_to_f64(bits)) <= tol)


@pytest.mark.parametrize("M,N,R", [(2320, 784, 528), (2576, 1808, 1040), (4112, 528, 144)])
@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1)])
def test_grouped_tile_order_every_element(M, N, R, fa, fb):
    """Shapes with more than 8 tile rows, so the tile order's 8-row raster
    groups engage and the last group is ragged (2320 = 9 tiles + 16 rows:
    groups of 8 and 2 tile rows; 2576: 11 tile rows; 4112: 17), with ragged
    tile columns and reductions; the tile count (40, 88, 51) is a multiple
    of 8 in the first two (the XCD remap engages) and not in the third.
    Every output element against the oracle, in every operand layout."""
    A, B = _operands(M, N, R, fa, fb, 5 * M + N + R + fa + 2 * fb)
    bits, _, tol = oracle.gemm_nt(A, FMT[fa], 6, B, FMT[fb], 11)
    want = oracle.bf16_to_f64(bits)
    for la, lb in [("rows", "rows")] + LAYOUTS:
        out = _run(A, fa, 6, B, fb, 11, la, lb)
        torch.cuda.synchronize()
        err = np.abs(oracle.bf16_to_f64(bf16_bits(out)) - want)
        bad = ~(err <= tol)
        assert not bad.any(), (la, lb, int(bad.sum()), np.argwhere(bad)[:4].tolist())
