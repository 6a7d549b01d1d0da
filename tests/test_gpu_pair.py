"""fp8_gemm_pair: a linear's dgrad and wgrad GEMMs in one launch, through
the C ABI.

[Perez et al. review, "Proposed method", bullets 3-4: the backward matmuls
run on the scaled FP8 operands, E5 gradients against E4 weights and
activations.] The pair kernel gives each output tile the single-GEMM
kernel's code for that tile, so both outputs must equal two separate
fp8_gemm calls bit for bit; one output per case is also checked against the
float64 oracle within the GEMM tolerance. Shapes cover partial tiles in
every dimension, tile counts of the first GEMM that are not multiples of
eight (the second GEMM's tiles then start mid-way through an XCD's range),
partial last stages, a second GEMM with R = 0, an empty member and the full
GPT-7B-style layer shapes."""
import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3, E5M2
import tensor_scaled_fp8_amd as tsf
from tests.gpu_util import bf16_bits, scale_record, to_dev_u8

pytestmark = pytest.mark.gpu


def _codes(shape, fmt, sigma, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return oracle.encode(g.standard_normal(shape) * sigma, fmt)


def _backward_operands(M, K, N, seed):
    """x8 [M,K] E4M3, w8 [K,N] E4M3, dy8 [M,N] E5M2 (row-major FP8 copies)."""
    x8 = _codes((M, K), E4M3, 40.0, seed)
    w8 = _codes((K, N), E4M3, 40.0, seed + 1)
    dy8 = _codes((M, N), E5M2, 1000.0, seed + 2)
    return x8, w8, dy8


def _pair_vs_single(x8, w8, dy8, bx, bw, bdy):
    M, K = x8.shape
    N = w8.shape[1]
    x, w, dy = to_dev_u8(x8), to_dev_u8(w8), to_dev_u8(dy8)
    sx, sw, sdy = scale_record(bx), scale_record(bw), scale_record(bdy)
    dgrad = dict(a=dy, fa="e5m2", sa=sdy, b=w, fb="e4m3", sb=sw)
    wgrad = dict(a=x, fa="e4m3", sa=sx, b=dy, fb="e5m2", sb=sdy, a_layout="cols", b_layout="cols")
    dX, dW = tsf.fp8_gemm_pair(dgrad, wgrad)
    dX1 = tsf.fp8_gemm(**dgrad)
    dW1 = tsf.fp8_gemm(**wgrad)
    torch.cuda.synchronize()
    assert tuple(dX.shape) == (M, K) and tuple(dW.shape) == (K, N)
    assert torch.equal(dX.view(torch.int16), dX1.view(torch.int16)), "dgrad differs from fp8_gemm"
    assert torch.equal(dW.view(torch.int16), dW1.view(torch.int16)), "wgrad differs from fp8_gemm"
    return dX, dW


@pytest.mark.parametrize("M,K,N", [(272, 528, 400), (256, 256, 256), (16, 16, 16), (784, 2064, 272),
                                   (48, 1040, 32), (512, 768, 3072), (1040, 784, 528)])
def test_pair_bit_identical_and_oracle(M, K, N):
    x8, w8, dy8 = _backward_operands(M, K, N, M + 3 * K + 7 * N)
    dX, dW = _pair_vs_single(x8, w8, dy8, 6, 11, 23)
    bits, _, tol = oracle.gemm_nt(dy8, E5M2, 23, np.ascontiguousarray(w8), E4M3, 11)
    err = np.abs(oracle.bf16_to_f64(bf16_bits(dX)) - oracle.bf16_to_f64(bits))
    assert not np.any(~(err <= tol)), float(np.max(err / tol))
    bits, _, tol = oracle.gemm_nt(np.ascontiguousarray(x8.T), E4M3, 6, np.ascontiguousarray(dy8.T), E5M2, 23)
    err = np.abs(oracle.bf16_to_f64(bf16_bits(dW)) - oracle.bf16_to_f64(bits))
    assert not np.any(~(err <= tol)), float(np.max(err / tol))


def test_pair_not_fusable_runs_both():
    """Two forward GEMMs (no one-launch kernel for that pair): two launches,
    same results as fp8_gemm."""
    a0, b0 = _codes((272, 400), E4M3, 40.0, 5), _codes((528, 400), E4M3, 40.0, 6)
    a1, b1 = _codes((48, 1040), E4M3, 40.0, 7), _codes((32, 1040), E4M3, 40.0, 8)
    g0 = dict(a=to_dev_u8(a0), fa="e4m3", sa=scale_record(6), b=to_dev_u8(b0), fb="e4m3", sb=scale_record(11))
    g1 = dict(a=to_dev_u8(a1), fa="e4m3", sa=scale_record(5), b=to_dev_u8(b1), fb="e4m3", sb=scale_record(12))
    y0, y1 = tsf.fp8_gemm_pair(g0, g1)
    r0, r1 = tsf.fp8_gemm(**g0), tsf.fp8_gemm(**g1)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), r0.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), r1.view(torch.int16))


def test_pair_with_empty_and_zero_reduction_members():
    """An empty second GEMM launches only the first; R = 0 (no tokens) in
    the wgrad gives dW = 0 while the dgrad is computed in the same launch."""
    x8, w8, dy8 = _backward_operands(272, 528, 400, 99)
    x, w, dy = to_dev_u8(x8), to_dev_u8(w8), to_dev_u8(dy8)
    sx, sw, sdy = scale_record(6), scale_record(11), scale_record(23)
    dgrad = dict(a=dy, fa="e5m2", sa=sdy, b=w, fb="e4m3", sb=sw)
    empty = dict(a=torch.empty((0, 0), dtype=torch.uint8, device="cuda"), fa="e4m3", sa=sx,
                 b=torch.empty((0, 0), dtype=torch.uint8, device="cuda"), fb="e5m2", sb=sdy,
                 a_layout="cols", b_layout="cols")
    dX, dW = tsf.fp8_gemm_pair(dgrad, empty)
    ref = tsf.fp8_gemm(**dgrad)
    torch.cuda.synchronize()
    assert dW.numel() == 0
    assert torch.equal(dX.view(torch.int16), ref.view(torch.int16))
    # wgrad over zero tokens: A [0, K] and B [0, N] read reduction-major
    zero_r = dict(a=torch.empty((0, 528), dtype=torch.uint8, device="cuda"), fa="e4m3", sa=sx,
                  b=torch.empty((0, 400), dtype=torch.uint8, device="cuda"), fb="e5m2", sb=sdy,
                  a_layout="cols", b_layout="cols",
                  out=torch.full((528, 400), 1.0, dtype=torch.bfloat16, device="cuda"))
    dX2, dW2 = tsf.fp8_gemm_pair(dgrad, zero_r)
    torch.cuda.synchronize()
    assert torch.equal(dX2.view(torch.int16), ref.view(torch.int16))
    assert not torch.any(dW2.view(torch.int16) != 0)


@pytest.mark.parametrize("name,M,K,N", [("qkv", 4096, 4096, 12288), ("proj", 4096, 4096, 4096),
                                        ("up", 4096, 4096, 16384), ("down", 4096, 16384, 4096)])
def test_pair_full_size_gpt7b_bit_identical(name, M, K, N):
    """The GPT-7B-style layer's backward pairs at full size (the launch the
    benchmark times): bit-identical to separate launches, and a sampled
    tile row of each output against the oracle."""
    g = torch.Generator(device="cuda")
    g.manual_seed(M + K + N)

    def codes(shape, sigma, dt):
        return (torch.randn(shape, device="cuda", generator=g) * sigma).to(dt).view(torch.uint8)
    x = codes((M, K), 40.0, torch.float8_e4m3fn)
    w = codes((K, N), 40.0, torch.float8_e4m3fn)
    dy = codes((M, N), 1000.0, torch.float8_e5m2)
    sx, sw, sdy = scale_record(6), scale_record(11), scale_record(23)
    dgrad = dict(a=dy, fa="e5m2", sa=sdy, b=w, fb="e4m3", sb=sw)
    wgrad = dict(a=x, fa="e4m3", sa=sx, b=dy, fb="e5m2", sb=sdy, a_layout="cols", b_layout="cols")
    dX, dW = tsf.fp8_gemm_pair(dgrad, wgrad)
    dX1 = tsf.fp8_gemm(**dgrad)
    dW1 = tsf.fp8_gemm(**wgrad)
    torch.cuda.synchronize()
    assert torch.equal(dX.view(torch.int16), dX1.view(torch.int16)), name
    assert torch.equal(dW.view(torch.int16), dW1.view(torch.int16)), name
    # oracle on the last 16 rows of each output (the last row of tiles)
    dy_h, w_h, x_h = dy.cpu().numpy(), w.cpu().numpy(), x.cpu().numpy()
    bits, _, tol = oracle.gemm_nt(dy_h[-16:], E5M2, 23, np.ascontiguousarray(w_h), E4M3, 11)
    err = np.abs(oracle.bf16_to_f64(bf16_bits(dX[-16:])) - oracle.bf16_to_f64(bits))
    assert not np.any(~(err <= tol)), (name, float(np.max(err / tol)))
    bits, _, tol = oracle.gemm_nt(np.ascontiguousarray(x_h[:, -16:].T), E4M3, 6,
                                  np.ascontiguousarray(dy_h.T), E5M2, 23)
    err = np.abs(oracle.bf16_to_f64(bf16_bits(dW[-16:])) - oracle.bf16_to_f64(bits))
    assert not np.any(~(err <= tol)), (name, float(np.max(err / tol)))


@pytest.mark.parametrize("M,K,N", [(2320, 784, 528), (528, 2576, 272)])
def test_pair_grouped_tile_order_every_element(M, K, N):
    """The backward pair on shapes whose dgrad or wgrad has more than 8 tile
    rows (ragged last raster group, ragged tiles and reductions): every
    element of both outputs against the oracle."""
    g = np.random.Generator(np.random.PCG64(M + 7 * K + 13 * N))
    x = oracle.encode(g.standard_normal((M, K)) * 40, E4M3)
    w = oracle.encode(g.standard_normal((K, N)) * 40, E4M3)
    dy = oracle.encode(g.standard_normal((M, N)) * 1000, E5M2)
    sx, sw, sdy = scale_record(6), scale_record(11), scale_record(23)
    xd, wd, dyd = (torch.from_numpy(a).cuda() for a in (x, w, dy))
    dgrad = dict(a=dyd, fa="e5m2", sa=sdy, b=wd, fb="e4m3", sb=sw)
    wgrad = dict(a=xd, fa="e4m3", sa=sx, b=dyd, fb="e5m2", sb=sdy, a_layout="cols", b_layout="cols")
    dX, dW = tsf.fp8_gemm_pair(dgrad, wgrad)
    torch.cuda.synchronize()
    for out, A, fa, ba, B, fb, bb in ((dX, dy, E5M2, 23, w, E4M3, 11),
                                      (dW, np.ascontiguousarray(x.T), E4M3, 6, np.ascontiguousarray(dy.T), E5M2, 23)):
        bits, _, tol = oracle.gemm_nt(A, fa, ba, B, fb, bb)
        err = np.abs(oracle.bf16_to_f64(bf16_bits(out)) - oracle.bf16_to_f64(bits))
        bad = ~(err <= tol)
        assert not bad.any(), (out.shape, int(bad.sum()), np.argwhere(bad)[:4].tolist())
