"""Seeded random sweep of fp8_gemm through the C ABI, against oracle.gemm_nt.

[Perez et al. review, "Proposed method", bullet 3: the matmul runs on the
scaled FP8 operands and the scaling is undone after it; bullet 4: E4 for
weights/activations, E5 for gradients.] Each case draws M, N, R (multiples
of 16, so tiles and the last k-stage are ragged in most cases), the two
formats, the two operand layouts and the two biases from a fixed seed, and
checks every output element against the float64 oracle within the GEMM
tolerance. The kernel has two tile bodies (the 16 x 16 x 128 MFMA one for a
row-layout A, the 32 x 32 x 64 one for a reduction-major A); each case also
runs the other layout of B, which takes the same body and must give the
same bits. Cases whose R is a multiple of 256 and whose E4M3 x E4M3 tiles
leave a last wave at most half full also run the tail split, which must
stay within the tolerance and change at most the tail tiles' bits.
"""
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
SEEDS = range(24)


def _case(seed):
    g = np.random.Generator(np.random.PCG64(1000 + seed))
    M, N = (int(16 * g.integers(1, 70)) for _ in range(2))
    R = int(16 * g.integers(1, 80)) if seed % 3 else int(256 * g.integers(1, 6))
    fa, fb = int(g.integers(0, 2)), int(g.integers(0, 2))
    la = "cols" if g.integers(0, 2) else "rows"
    lb = "cols" if g.integers(0, 2) else "rows"
    ba, bb = int(g.integers(-4, 12)), int(g.integers(-4, 12))
    sig = (6.0, 40.0, 1e3)
    A = oracle.encode(g.standard_normal((M, R)) * sig[int(g.integers(0, 3))], FMT[fa])
    B = oracle.encode(g.standard_normal((N, R)) * sig[int(g.integers(0, 3))], FMT[fb])
    return M, N, R, fa, fb, la, lb, ba, bb, A, B


def _run(A, fa, ba, B, fb, bb, la, lb, **kw):
    a = to_dev_u8(np.ascontiguousarray(A.T) if la == "cols" else A)
    b = to_dev_u8(np.ascontiguousarray(B.T) if lb == "cols" else B)
    return tsf.fp8_gemm(a, NAME[fa], scale_record(ba), b, NAME[fb], scale_record(bb), a_layout=la, b_layout=lb,
                        **kw)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_gemm_against_oracle(seed):
    M, N, R, fa, fb, la, lb, ba, bb, A, B = _case(seed)
    print(f"\n[sweep] seed {seed}: M={M} N={N} R={R} {NAME[fa]}x{NAME[fb]} {la}/{lb} biases {ba},{bb}", flush=True)
    bits, _, tol = oracle.gemm_nt(A, FMT[fa], ba, B, FMT[fb], bb)
    want = oracle.bf16_to_f64(bits)
    out = _run(A, fa, ba, B, fb, bb, la, lb)
    other = _run(A, fa, ba, B, fb, bb, la, "rows" if lb == "cols" else "cols")
    torch.cuda.synchronize()
    err = np.abs(oracle.bf16_to_f64(bf16_bits(out)) - want)
    bad = ~(err <= tol)
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:4].tolist())
    assert torch.equal(out.view(torch.int16), other.view(torch.int16))
    if fa == 0 and fb == 0:
        nb = tsf.gemm_workspace_bytes("e4m3", "e4m3", M, N, R, "tail")
        if nb:
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            split = _run(A, fa, ba, B, fb, bb, la, lb, workspace=ws, split="tail")
            torch.cuda.synchronize()
            err = np.abs(oracle.bf16_to_f64(bf16_bits(split)) - want)
            bad = ~(err <= tol)
            assert not bad.any(), ("split", int(bad.sum()))
            ntail = nb // (2 * 65536 * 4)
            diff = (split.view(torch.int16) != out.view(torch.int16)).cpu().numpy()
            tm, tn = (M + 255) // 256, (N + 255) // 256
            tiles = np.zeros((tm, tn), bool)
            for i, j in np.argwhere(diff):
                tiles[i // 256, j // 256] = True
            assert tiles.sum() <= ntail, (int(tiles.sum()), ntail)
