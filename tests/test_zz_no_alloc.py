"""fp8_gemm_noalloc (the GEMM whose tail-split partials live in the
library's own device scratch, for callers that cannot allocate) through the
C ABI, against fp8_gemm_ws with a caller workspace: the same kernels, so
the outputs must be bit-identical; and against the oracle within the GEMM
tolerance. Two calls in a row on one device, the second smaller, so the
second runs on the scratch contents the first left."""
import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3
import tensor_scaled_fp8_amd as tsf
from tests.gpu_util import bf16_bits, scale_record, to_dev_u8

pytestmark = pytest.mark.gpu


def _case(M, N, R, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    A = oracle.encode(g.standard_normal((M, R)) * 40, E4M3)
    B = oracle.encode(g.standard_normal((R, N)) * 40, E4M3)     # reduction-major, as the forward reads w8
    return A, B


def _check(M, N, R, seed, split):
    A, B = _case(M, N, R, seed)
    a, b = to_dev_u8(A), to_dev_u8(B)
    sa, sb = scale_record(6), scale_record(11)
    nbytes = tsf.gemm_workspace_bytes("e4m3", "e4m3", M, N, R, split)
    assert 0 < nbytes <= tsf.FP8_NOALLOC_SCRATCH_BYTES, nbytes     # the shape does split
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ref = tsf.fp8_gemm(a, "e4m3", sa, b, "e4m3", sb, a_layout="rows", b_layout="cols", workspace=ws, split=split)
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    tsf.fp8_gemm_noalloc(a, "e4m3", sa, b, "e4m3", sb, out, "rows", "cols", split=split)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (M, N, R, split)
    bits, _, tol = oracle.gemm_nt(A, E4M3, 6, np.ascontiguousarray(B.T), E4M3, 11)
    err = np.abs(oracle.bf16_to_f64(bf16_bits(out)) - oracle.bf16_to_f64(bits))
    assert not np.any(~(err <= tol)), (M, N, R, float(np.max(err / tol)))


def test_noalloc_matches_workspace_gemm_two_calls():
    # 384 tiles of 256 x 256 on 256 CUs: 128 tail tiles, the scratch's full size
    _check(2048, 12288, 1024, 1, "tail")
    # then a smaller one: 12 tiles, all split, over the first call's leftovers
    _check(784, 528, 2048, 2, "tail")


def test_noalloc_without_split_and_auto():
    """No split (NEVER, or AUTO at a short reduction): plain fp8_gemm output."""
    M, N, R = 528, 272, 1040
    A, B = _case(M, N, R, 3)
    a, b = to_dev_u8(A), to_dev_u8(B)
    sa, sb = scale_record(6), scale_record(11)
    ref = tsf.fp8_gemm(a, "e4m3", sa, b, "e4m3", sb, a_layout="rows", b_layout="cols")
    for split in ("never", "auto"):
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        tsf.fp8_gemm_noalloc(a, "e4m3", sa, b, "e4m3", sb, out, "rows", "cols", split=split)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), split
