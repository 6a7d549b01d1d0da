"""Out-of-bounds writes: every output buffer of the hot-path entry points
sits between guard bands of a known byte, on ragged shapes (partial tiles
in every dimension); after the calls the guards must be intact. Records,
FP8 copies, bf16 GEMM outputs and the split GEMM's workspace are all
guarded. The values themselves are checked by the parity tests."""
import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3, E5M2
import tensor_scaled_fp8_amd as tsf
from tests.gpu_util import to_dev_bf16, to_dev_u8
from workloads import draw_normal_bf16

pytestmark = pytest.mark.gpu
PAD = 4096
CANARY = 0xA5


class Guarded:
    """A device buffer with guard bands; .t is the 16-B aligned view."""

    def __init__(self, shape, dtype):
        self.n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((PAD + self.n + PAD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[PAD:PAD + self.n].view(dtype).view(shape)

    def intact(self):
        torch.cuda.synchronize()
        b = self.buf.cpu().numpy()
        return bool(np.all(b[:PAD] == CANARY) and np.all(b[PAD + self.n:] == CANARY))


def _record():
    g = Guarded((16,), torch.int32)
    g.t.zero_()
    return g


def test_quantize_cast_outputs_guarded():
    rows, cols = 272, 400
    x = to_dev_bf16(draw_normal_bf16(1, (rows, cols), 1.0))
    s = _record()
    rw, tr = Guarded((rows, cols), torch.uint8), Guarded((cols, rows), torch.uint8)
    tsf.fp8_quantize(x, "e4m3", s.t, out_row=rw.t, out_t=tr.t)
    assert s.intact() and rw.intact() and tr.intact()
    rw2, tr2 = Guarded((rows, cols), torch.uint8), Guarded((cols, rows), torch.uint8)
    tsf.fp8_cast(x, "e5m2", s.t, out_row=rw2.t, out_t=tr2.t)
    assert rw2.intact() and tr2.intact()


def test_quantize_batch_outputs_guarded():
    shapes = [(272, 400), (48, 1040), (16, 16)]
    xs = [to_dev_bf16(draw_normal_bf16(10 + i, sh, 1.0)) for i, sh in enumerate(shapes)]
    recs = [_record() for _ in shapes]
    outs = [(Guarded(sh, torch.uint8), Guarded(sh[::-1], torch.uint8)) for sh in shapes]
    tsf.fp8_quantize_batch([dict(x=x, fmt="e4m3" if i % 2 == 0 else "e5m2", s=recs[i].t, out_row=o[0].t,
                                 out_t=o[1].t) for i, (x, o) in enumerate(zip(xs, outs))])
    for r, (a, b) in zip(recs, outs):
        assert r.intact() and a.intact() and b.intact()


@pytest.mark.parametrize("la,lb", [("rows", "rows"), ("rows", "cols"), ("cols", "rows"), ("cols", "cols")])
def test_gemm_outputs_guarded(la, lb):
    M, N, R = 784, 272, 400
    g = np.random.Generator(np.random.PCG64(3))
    A = oracle.encode(g.standard_normal((M, R)) * 6, E4M3)
    B = oracle.encode(g.standard_normal((N, R)) * 40, E4M3)
    a = to_dev_u8(np.ascontiguousarray(A.T) if la == "cols" else A)
    b = to_dev_u8(np.ascontiguousarray(B.T) if lb == "cols" else B)
    sa, sb = _record(), _record()
    sa.t[1] = 6
    sb.t[1] = 11
    C = Guarded((M, N), torch.bfloat16)
    tsf.fp8_gemm(a, "e4m3", sa.t, b, "e4m3", sb.t, out=C.t, a_layout=la, b_layout=lb)
    assert C.intact() and sa.intact() and sb.intact()


def test_pair_and_split_outputs_guarded():
    M, K, N = 272, 528, 400
    g = np.random.Generator(np.random.PCG64(4))
    x8 = to_dev_u8(oracle.encode(g.standard_normal((M, K)) * 6, E4M3))
    w8 = to_dev_u8(oracle.encode(g.standard_normal((K, N)) * 40, E4M3))
    dy8 = to_dev_u8(oracle.encode(g.standard_normal((M, N)) * 1e3, E5M2))
    sx, sw, sdy = _record(), _record(), _record()
    dX, dW = Guarded((M, K), torch.bfloat16), Guarded((K, N), torch.bfloat16)
    tsf.fp8_gemm_pair(dict(a=dy8, fa="e5m2", sa=sdy.t, b=w8, fb="e4m3", sb=sw.t, out=dX.t),
                      dict(a=x8, fa="e4m3", sa=sx.t, b=dy8, fb="e5m2", sb=sdy.t, out=dW.t,
                           a_layout="cols", b_layout="cols"))
    assert dX.intact() and dW.intact()
    # tail split: output and workspace guarded (R = 1024, ragged M and N)
    A = to_dev_u8(oracle.encode(g.standard_normal((M, 1024)) * 6, E4M3))
    Bm = to_dev_u8(oracle.encode(g.standard_normal((N, 1024)) * 40, E4M3))
    nb = tsf.gemm_workspace_bytes("e4m3", "e4m3", M, N, 1024, "tail")
    assert nb > 0
    ws = Guarded((nb,), torch.uint8)
    C = Guarded((M, N), torch.bfloat16)
    tsf.fp8_gemm(A, "e4m3", sx.t, Bm, "e4m3", sw.t, out=C.t, workspace=ws.t, split="tail")
    assert C.intact() and ws.intact()


def test_wgrad_fp8_outputs_guarded():
    M, K, N = 400, 272, 528
    g = np.random.Generator(np.random.PCG64(5))
    x8 = to_dev_u8(oracle.encode(g.standard_normal((M, K)) * 6, E4M3))
    dy8 = to_dev_u8(oracle.encode(g.standard_normal((M, N)) * 1e3, E5M2))
    sx, sdy, sdw = _record(), _record(), _record()
    sx.t[1] = 6
    sdy.t[1] = 23
    dW = Guarded((K, N), torch.bfloat16)
    dw8, dw8t = Guarded((K, N), torch.uint8), Guarded((N, K), torch.uint8)
    tsf.fp8_wgrad_fp8(x8, sx.t, dy8, sdy.t, 0, 0, dW=dW.t, s_dw=sdw.t, dw8=dw8.t, dw8t=dw8t.t, transposed=True,
                      x_layout="cols", dy_layout="cols")
    assert dW.intact() and dw8.intact() and dw8t.intact() and sdw.intact()
