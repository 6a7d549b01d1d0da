"""GPU parity of each hot-path step against the oracle, through the C ABI.

Bar: amax, bias, scale, flags and every FP8 byte bit-exact; GEMM outputs
within |C - C_oracle| <= 1 bf16 ulp + 1e-4 * 2^-(ba+bb) * sum_r |a_r b_r|."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3, E5M2
import tensor_scaled_fp8_amd as tsf
from tests.gpu_util import bf16_bits, f32_bits, scale_record, to_dev_bf16, to_dev_u8, u8
from workloads import draw_normal_bf16, f32_to_bf16_bits, random_bf16_bits

pytestmark = pytest.mark.gpu
FMT = {0: E4M3, 1: E5M2}
NAME = {0: "e4m3", 1: "e5m2"}


def _check_record(rec, bits, fmt_id, margin, mu, fused=True):
    a = oracle.amax(bits)
    if math.isnan(a):
        assert math.isnan(rec["amax"]) and rec["gen_max"] & 0xFFFF > 0x7F80
    else:
        assert f32_bits(rec["amax"]) == f32_bits(a), (rec["amax"], a)
        assert rec["gen_max"] & 0xFFFF == f32_bits(a) >> 16
    assert rec["reduce_bits"] == 0
    if fused:
        b, fl = oracle.compute_bias(a, FMT[fmt_id], margin, mu)
        assert (rec["bias"], rec["flags"]) == (b, fl), (rec, b, fl)
        assert rec["scale"] == 2.0 ** b and rec["scale_inv"] == 2.0 ** -b


# ---------------------------------------------------------------- a1 / a2
@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 4096, 65536 + 5, 1 << 20, 3_000_017])
def test_amax_sizes(n):
    bits = random_bf16_bits(100 + n, (n,))
    s = tsf.new_scale(1)[0]
    x = to_dev_bf16(bits)
    tsf.fp8_amax_scale(x, "e4m3", s)
    _check_record(tsf.read_scale(s), bits, 0, 0, 0)
    tsf.fp8_amax(x, s)   # unfused: amax + flags only, bias 0
    r = tsf.read_scale(s)
    _check_record(r, bits, 0, 0, 0, fused=False)
    assert r["bias"] == 0 and r["scale"] == 1.0


def test_amax_special_tensors():
    n = 1 << 18
    cases = {
        "zeros": np.zeros(n, np.uint16),
        "neg_zeros": np.full(n, 0x8000, np.uint16),
        "spike_last": np.zeros(n, np.uint16),
        "spike_first": np.zeros(n, np.uint16),
        "tiny_subnormal": np.full(n, 0x0001, np.uint16),
        "max_finite": draw_normal_bf16(3, (n,), 1.0),
        "inf": draw_normal_bf16(4, (n,), 1.0),
        "nan": draw_normal_bf16(5, (n,), 1.0),
        "nan_and_inf": draw_normal_bf16(6, (n,), 1.0),
    }
    cases["spike_last"][-1] = 0xC2F6        # -123
    cases["spike_first"][0] = 0x4480        # 1024
    cases["max_finite"][777] = 0xFF7F
    cases["inf"][1234] = 0xFF80
    cases["nan"][99] = 0x7FC1
    cases["nan_and_inf"][5] = 0x7F80
    cases["nan_and_inf"][6] = 0xFFFF
    for name, bits in cases.items():
        for fmt_id in (0, 1):
            s = tsf.new_scale(1)[0]
            tsf.fp8_amax_scale(to_dev_bf16(bits), NAME[fmt_id], s, margin=1, mu_log2=2 * fmt_id)
            _check_record(tsf.read_scale(s), bits, fmt_id, 1, 2 * fmt_id)


def test_amax_reduction_state_reused():
    """The same record serves many calls in a row (state returns to zero)."""
    s = tsf.new_scale(1)[0]
    for k in range(6):
        bits = draw_normal_bf16(50 + k, (1 << 16) + 16 * k, 10.0 ** (k - 3))
        tsf.fp8_amax_scale(to_dev_bf16(bits), "e5m2", s)
        _check_record(tsf.read_scale(s), bits, 1, 0, 0)


def test_scale_kernel_rule_spot_values():
    g = np.random.Generator(np.random.PCG64(9))
    vals = list(oracle.bf16_to_f64(g.integers(1, 0x7F80, 300).astype(np.uint16))) + [
        448.0, 450.0, 1.0, 2.0 ** -133, 57344.0, 0.0, math.inf, math.nan]
    recs = tsf.new_scale(len(vals))
    for i, a in enumerate(vals):
        recs[i] = scale_record(0, 0, float(a))
    for fmt_id, margin, mu in ((0, 0, 0), (1, 1, -2), (0, -3, 0), (1, 0, 5)):
        for i in range(len(vals)):
            tsf.fp8_scale(NAME[fmt_id], recs[i], margin, mu)
        host = recs.cpu()
        for i, a in enumerate(vals):
            w = host[i]
            b, fl = oracle.compute_bias(float(a), FMT[fmt_id], margin, mu)
            assert (int(w[1]), int(w[4])) == (b, fl), (a, fmt_id, margin, mu)
            assert float(w.view(torch.float32)[2]) == 2.0 ** b


# ---------------------------------------------------------------- a3 cast
ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)


@pytest.mark.parametrize("fmt_id", [0, 1])
def test_cast_exhaustive_all_bf16_all_biases(fmt_id):
    """All 65536 bf16 patterns (NaN, inf, subnormals, +-0) x every bias in
    [-126, 126], row-wise and transposed outputs."""
    x = to_dev_bf16(ALL_BF16)
    row = torch.empty((256, 256), dtype=torch.uint8, device="cuda")
    tr = torch.empty((256, 256), dtype=torch.uint8, device="cuda")
    xf = oracle.bf16_to_f64(ALL_BF16)
    for b in range(-126, 127):
        s = scale_record(b, flags=tsf.FLAG_NONFINITE)
        tsf.fp8_cast(x, NAME[fmt_id], s, row, tr)
        want = oracle.encode(np.ldexp(xf, b), FMT[fmt_id])
        got = u8(row)
        bad = np.argwhere(got != want)
        assert bad.size == 0, (b, [(hex(ALL_BF16[i, j]), hex(got[i, j]), hex(want[i, j])) for i, j in bad[:8]])
        assert np.array_equal(u8(tr), want.T), b


@pytest.mark.parametrize("fmt_id", [0, 1])
def test_cast_fast_path_finite_tensor(fmt_id):
    """Without the NONFINITE flag (no NaN in the tensor): every finite and
    infinite bf16 pattern, a spread of biases."""
    bits = ALL_BF16.copy()
    nan = (bits & 0x7FFF) > 0x7F80
    bits[nan] = 0x3F80
    x = to_dev_bf16(bits)
    xf = oracle.bf16_to_f64(bits)
    for b in (-126, -40, -7, -1, 0, 1, 6, 12, 23, 29, 60, 126):
        rw, tr = tsf.fp8_cast(x, NAME[fmt_id], scale_record(b))
        want = oracle.encode(np.ldexp(xf, b), FMT[fmt_id])
        assert np.array_equal(u8(rw), want) and np.array_equal(u8(tr), want.T), b


@pytest.mark.parametrize("shape", [(16, 16), (16, 4096), (144, 272), (528, 1040), (128, 128),
                                   (256, 384), (1024, 48), (2064, 784)])
def test_cast_shapes_ragged_tiles(shape):
    bits = draw_normal_bf16(shape[0] * 7 + shape[1], shape, 0.37)
    x = to_dev_bf16(bits)
    for fmt_id in (0, 1):
        s = tsf.new_scale(1)[0]
        tsf.fp8_amax_scale(x, NAME[fmt_id], s)
        rec = oracle.scale_record(bits, FMT[fmt_id])
        rw, tr = tsf.fp8_cast(x, NAME[fmt_id], s)
        q, qt = oracle.cast(bits, FMT[fmt_id], rec["bias"])
        assert np.array_equal(u8(rw), q) and np.array_equal(u8(tr), qt)
        # single-output modes, with canaries around the buffers
        buf = torch.full((shape[0] * shape[1] + 64,), 0xA5, dtype=torch.uint8, device="cuda")
        out = buf[16:16 + shape[0] * shape[1]].view(shape[1], shape[0])
        tsf.fp8_cast(x, NAME[fmt_id], s, out_row=None, out_t=out, rowwise=False)
        hb = u8(buf)
        assert np.array_equal(hb[16:16 + q.size].reshape(shape[1], shape[0]), qt)
        assert np.all(hb[:16] == 0xA5) and np.all(hb[16 + q.size:] == 0xA5)
        rw2, none = tsf.fp8_cast(x, NAME[fmt_id], s, transposed=False)
        assert none is None and np.array_equal(u8(rw2), q)


def test_cast_empty():
    x = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    rw, tr = tsf.fp8_cast(x, "e4m3", scale_record(3))
    assert rw.shape == (0, 32) and tr.shape == (32, 0)


# ---------------------------------------------------------------- a4-a6 GEMM
def _finite_codes(fmt):
    t = oracle.decode_table(fmt)
    return np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)


def _gemm_check(A, fa, ba, B, fb, bb, exact=False):
    out = tsf.fp8_gemm_nt(to_dev_u8(A), NAME[fa], scale_record(ba), to_dev_u8(B), NAME[fb],
                          scale_record(bb))
    got = oracle.bf16_to_f64(bf16_bits(out))
    bits, c64, tol = oracle.gemm_nt(A, FMT[fa], ba, B, FMT[fb], bb)
    if exact:
        assert np.array_equal(bf16_bits(out), bits)
    err = np.abs(got - oracle.bf16_to_f64(bits))
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, [(i, j, got[i, j], c64[i, j], tol[i, j]) for i, j in bad[:8]]
    return got, c64


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_gemm_brute_force_small(fa, fb):
    g = np.random.Generator(np.random.PCG64(31 + 4 * fa + fb))
    for M, N, R in ((16, 16, 16), (32, 32, 64), (48, 80, 144), (32, 64, 128)):
        A = g.choice(_finite_codes(FMT[fa]), size=(M, R))
        B = g.choice(_finite_codes(FMT[fb]), size=(N, R))
        _gemm_check(A, fa, 3, B, fb, 7)


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1)])
def test_gemm_one_hot_exact(fa, fb):
    """B = permutation of 1.0 codes: C reproduces columns of A exactly, so
    the k pairing, the output layout and the epilogue scale are pinned
    bit for bit (including FP8 subnormals, which must not be flushed)."""
    g = np.random.Generator(np.random.PCG64(77))
    for M, R in ((32, 64), (288, 320), (16, 16)):
        A = g.choice(_finite_codes(FMT[fa]), size=(M, R))
        one = int(oracle.encode(np.array([1.0]), FMT[fb])[0])
        perm = g.permutation(R)
        B = np.zeros((R, R), np.uint8)
        B[np.arange(R), perm] = one
        _gemm_check(A, fa, 2, B, fb, -1, exact=True)


def test_gemm_subnormal_operands():
    g = np.random.Generator(np.random.PCG64(5))
    sub4 = np.array([c for c in range(1, 8)] + [0x80 | c for c in range(1, 8)], np.uint8)
    sub5 = np.array([1, 2, 3, 0x81, 0x82, 0x83], np.uint8)
    A = g.choice(sub4, size=(64, 128))
    B = g.choice(sub5, size=(96, 128))
    got, c64 = _gemm_check(A, 0, 0, B, 1, 0)
    assert np.count_nonzero(got) > 0.9 * got.size


@pytest.mark.parametrize("M,N,R", [(272, 528, 400), (512, 3072, 768), (256, 256, 128),
                                   (784, 272, 2064), (16, 1040, 528)])
def test_gemm_ragged_multi_tile(M, N, R):
    g = np.random.Generator(np.random.PCG64(M + N + R))
    for fa, fb in ((0, 0), (1, 0), (0, 1)):
        A = oracle.encode(g.standard_normal((M, R)) * 40, FMT[fa])
        B = oracle.encode(g.standard_normal((N, R)) * 40, FMT[fb])
        _gemm_check(A, fa, 6, B, fb, 11)


def test_gemm_extremes_saturated_operands():
    """+-max codes everywhere: large sums, and the epilogue's 2^-(ba+bb)."""
    g = np.random.Generator(np.random.PCG64(6))
    A = np.where(g.random((64, 256)) < 0.5, 0x7E, 0xFE).astype(np.uint8)
    B = np.where(g.random((64, 256)) < 0.5, 0x7B, 0xFB).astype(np.uint8)
    _gemm_check(A, 0, 20, B, 1, 30)


@pytest.mark.parametrize("shift", [-252, -140, -95, -94, -60, 0, 40, 72, 73, 100])
@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_gemm_dequant_scale_range(shift, fa, fb):
    """2^-(ba+bb) across the whole bias range (around [-94, 72], where the
    scaling could also be folded into the MFMA operand scales exactly):
    outputs that underflow to zero, land on bf16 subnormals, or sit near the
    top of the bf16 range all follow the oracle's single rounding."""
    g = np.random.Generator(np.random.PCG64(1000 + shift + 4 * fa + fb))
    ba = -shift // 2
    bb = -shift - ba
    A = g.choice(_finite_codes(FMT[fa]), size=(80, 320))
    B = g.choice(_finite_codes(FMT[fb]), size=(48, 320))
    if shift >= 72:   # keep |C| below the bf16 maximum
        A = np.where(np.abs(oracle.decode_table(FMT[fa])[A]) > 4, 0, A).astype(np.uint8)
        B = np.where(np.abs(oracle.decode_table(FMT[fb])[B]) > 4, 0, B).astype(np.uint8)
    _gemm_check(A, fa, ba, B, fb, bb)


def test_gemm_degenerate():
    s = scale_record(0)
    a = torch.zeros((32, 0), dtype=torch.uint8, device="cuda")
    b = torch.zeros((48, 0), dtype=torch.uint8, device="cuda")
    c = torch.full((32, 48), 7.0, dtype=torch.bfloat16, device="cuda")
    tsf.fp8_gemm_nt(a, "e4m3", s, b, "e4m3", s, out=c)
    assert torch.all(c == 0)
    e = tsf.fp8_gemm_nt(torch.zeros((0, 64), dtype=torch.uint8, device="cuda"), "e4m3", s,
                        torch.zeros((16, 64), dtype=torch.uint8, device="cuda"), "e4m3", s)
    assert e.shape == (0, 16)


# ---------------------------------------------------------------- composed linear
@pytest.mark.parametrize("M,K,N,margin,mu", [(512, 768, 3072, 0, 0), (272, 400, 528, 1, -1),
                                             (64, 128, 48, 0, 3)])
@pytest.mark.parametrize("transposed", [False, True])
def test_linear_fwd_bwd_vs_oracle(M, K, N, margin, mu, transposed):
    """The GEMMs read the row-major FP8 copies (reduction-major where
    needed); the transposed copies are written only when the workspace
    has them, and then match the oracle too."""
    X = draw_normal_bf16(1, (M, K), 1.0)
    W = draw_normal_bf16(2, (K, N), 0.02)
    dY = draw_normal_bf16(3, (M, N), 1e-4)
    ws = tsf.LinearWorkspace(M, K, N, transposed=transposed)
    Y = tsf.fp8_linear_fwd(to_dev_bf16(X), to_dev_bf16(W), ws, margin)
    dX, dW = tsf.fp8_linear_bwd(to_dev_bf16(dY), ws, margin, mu)
    ref = oracle.linear_fwd_bwd(X, W, dY, margin, mu)
    for key, s in (("sx", ws.sx), ("sw", ws.sw), ("sdy", ws.sdy)):
        r = tsf.read_scale(s)
        assert f32_bits(r["amax"]) == f32_bits(ref[key]["amax"])
        assert (r["bias"], r["flags"]) == (ref[key]["bias"], ref[key]["flags"]), key
    for key in ("x8", "x8t", "w8", "w8t", "dy8", "dy8t") if transposed else ("x8", "w8", "dy8"):
        assert np.array_equal(u8(getattr(ws, key)), ref[key]), key
    for key, t in (("Y", Y), ("dX", dX), ("dW", dW)):
        bits, c64, tol = ref[key]
        err = np.abs(oracle.bf16_to_f64(bf16_bits(t)) - oracle.bf16_to_f64(bits))
        assert np.all(err <= tol), (key, float((err / tol).max()))


def test_autograd_linear_module():
    torch.manual_seed(0)
    lin = tsf.Linear(256, 384, device="cuda")
    x = (torch.randn(2, 64, 256, device="cuda")).to(torch.bfloat16).requires_grad_(True)
    y = lin(x)
    assert y.shape == (2, 64, 384) and y.dtype == torch.bfloat16
    y.backward(torch.randn_like(y) * 1e-3)
    assert x.grad.shape == x.shape and lin.weight.grad.shape == lin.weight.shape
    ref = x.detach().float() @ lin.weight.detach().float()
    rel = (y.float() - ref).norm() / ref.norm()
    assert rel < 0.08


def test_autograd_linear_reuses_workspace_and_matches_oracle():
    """Training-loop use of the drop-in module: after the first step the
    forward takes a free workspace from the pool (no new device buffers),
    and every step's Y, dX and dW are the oracle's within the GEMM
    tolerance, with the FP8 copies of that step's inputs."""
    tsf.release_workspaces()
    M, K, N, margin, mu = 128, 256, 384, 1, 2
    lin = tsf.Linear(K, N, margin=margin, mu_log2=mu, device="cuda")
    wb = bf16_bits(lin.weight.detach())
    seen = []
    for step in range(4):
        xb = draw_normal_bf16(900 + step, (M, K), 1.0)
        dyb = draw_normal_bf16(950 + step, (M, N), 1e-5)
        x = to_dev_bf16(xb).requires_grad_(True)
        lin.weight.grad = None
        y = lin(x)
        ws = y.grad_fn.lease.ws
        seen.append(tuple(t.data_ptr() for t in (ws.x8, ws.w8, ws.dy8, ws.scales)))
        y.backward(to_dev_bf16(dyb))
        torch.cuda.synchronize()
        ref = oracle.linear_fwd_bwd(xb, wb, dyb, margin, mu)
        for key, t in (("Y", y), ("dX", x.grad), ("dW", lin.weight.grad)):
            bits, c64, tol = ref[key]
            err = np.abs(oracle.bf16_to_f64(bf16_bits(t)) - oracle.bf16_to_f64(bits))
            assert np.all(err <= tol), (step, key, float((err / tol).max()))
        del y, x
    # steps 1.. reuse the workspace step 0 built (its graph freed before the next forward)
    assert len(set(seen)) == 1, seen
    tsf.release_workspaces()


# ---------------------------------------------------------------- a1+a2+a3 fused
@pytest.mark.parametrize("shape", [(16, 16), (144, 272), (528, 1040), (2064, 784)])
@pytest.mark.parametrize("fmt_id,margin,mu", [(0, 0, 0), (1, 1, -2), (1, 0, 3), (0, 2, 0)])
def test_quantize_matches_oracle(shape, fmt_id, margin, mu):
    bits = draw_normal_bf16(shape[0] * 13 + shape[1] + fmt_id, shape, 0.02 if fmt_id == 0 else 1e-5)
    x = to_dev_bf16(bits)
    s = tsf.new_scale(1)[0]
    rw, tr = tsf.fp8_quantize(x, NAME[fmt_id], s, margin, mu)
    _check_record(tsf.read_scale(s), bits, fmt_id, margin, mu)
    rec = oracle.scale_record(bits, FMT[fmt_id], margin, mu)
    q, qt = oracle.cast(bits, FMT[fmt_id], rec["bias"])
    assert np.array_equal(u8(rw), q) and np.array_equal(u8(tr), qt)


def test_quantize_special_tensors_and_outputs():
    n = 256
    base = draw_normal_bf16(21, (n, n), 1.0)
    cases = {"zeros": np.zeros((n, n), np.uint16), "nan": base.copy(), "inf": base.copy(),
             "tiny": np.full((n, n), 0x0001, np.uint16)}
    cases["nan"][3, 5] = 0xFFC1
    cases["inf"][200, 7] = 0x7F80
    for name, bits in cases.items():
        for fmt_id in (0, 1):
            s = tsf.new_scale(1)[0]
            rw, tr = tsf.fp8_quantize(to_dev_bf16(bits), NAME[fmt_id], s)
            _check_record(tsf.read_scale(s), bits, fmt_id, 0, 0)
            rec = oracle.scale_record(bits, FMT[fmt_id])
            q, qt = oracle.cast(bits, FMT[fmt_id], rec["bias"])
            assert np.array_equal(u8(rw), q) and np.array_equal(u8(tr), qt), name
    # single-output and no-output forms still publish the record
    s = tsf.new_scale(1)[0]
    rw, none = tsf.fp8_quantize(to_dev_bf16(base), "e4m3", s, transposed=False)
    assert none is None
    _check_record(tsf.read_scale(s), base, 0, 0, 0)
    s = tsf.new_scale(1)[0]
    tsf.fp8_quantize(to_dev_bf16(base), "e5m2", s, rowwise=False, transposed=False)
    _check_record(tsf.read_scale(s), base, 1, 0, 0)
    s = tsf.new_scale(1)[0]
    tsf.fp8_quantize(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), "e4m3", s)
    r = tsf.read_scale(s)
    assert r["amax"] == 0.0 and r["flags"] == tsf.FLAG_ZERO and r["bias"] == 0


def test_quantize_repeated_calls_shrinking_amax():
    """The generation-tagged running max must not keep an earlier call's
    larger maximum; interleaving with the standalone amax path on the same
    record keeps both correct."""
    s = tsf.new_scale(1)[0]
    for k, sigma in enumerate((100.0, 1.0, 1e-3, 50.0, 1e-6, 2.0)):
        bits = draw_normal_bf16(300 + k, (128, 256), sigma)
        x = to_dev_bf16(bits)
        rw, _ = tsf.fp8_quantize(x, "e4m3", s, transposed=False)
        _check_record(tsf.read_scale(s), bits, 0, 0, 0)
        rec = oracle.scale_record(bits, E4M3)
        assert np.array_equal(u8(rw), oracle.cast(bits, E4M3, rec["bias"])[0])
        if k % 2:
            tsf.fp8_amax_scale(x, "e5m2", s, 1, 0)
            _check_record(tsf.read_scale(s), bits, 1, 1, 0)
