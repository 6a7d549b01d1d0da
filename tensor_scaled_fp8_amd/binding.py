"""Thin Python binding over the C ABI (include/fp8lin.h): argument
marshalling only. Torch supplies device memory and the current HIP stream;
every step of the computation runs in the HIP kernels of libfp8lin.so.

Names follow the C entry points: fp8_amax, fp8_scale, fp8_amax_scale,
fp8_scale_fixed, fp8_cast, fp8_gemm_nt, fp8_gemm, fp8_gemm_pair, fp8_quantize, fp8_quantize_batch,
fp8_quantize_spec,
fp8_linear_fwd,
fp8_linear_bwd, fp8_linear_fwd_cached, fp8_wgrad_fp8, fp8_adam_init_master,
fp8_adam_step. A scaling record (fp8_scale_t, 64
bytes) is an int32 tensor of 16 words on the device."""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import (FP8_E4M3, FP8_E5M2, FP8_OPERAND_COLS, FP8_OPERAND_ROWS, FP8_SCALING_AMAX, FP8_SCALING_FIXED,
                   FP8_SPLIT_AUTO, FP8_SPLIT_NEVER, FP8_SPLIT_TAIL,
                   GemmArgs, LinearWs, QuantizeArgs, check, load)

SCALE_WORDS = 16         # sizeof(fp8_scale_t) / 4
SCALINGS = {"amax": FP8_SCALING_AMAX, "fixed": FP8_SCALING_FIXED}
FMT_CODES = {"e4m3": FP8_E4M3, "e5m2": FP8_E5M2, FP8_E4M3: FP8_E4M3, FP8_E5M2: FP8_E5M2}


def _fmt(f) -> int:
    try:
        return FMT_CODES[f]
    except KeyError:
        raise ValueError(f"unknown FP8 format {f!r}") from None


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: Optional[torch.Tensor], dtype, name: str) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (no CPU path exists)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def new_scale(count: int = 1, device="cuda") -> torch.Tensor:
    """Zeroed scaling record(s): int32 [count, 16]."""
    return torch.zeros((count, SCALE_WORDS), dtype=torch.int32, device=device)


def read_scale(s: torch.Tensor) -> dict:
    """Copy a record to the host (synchronises) and decode its fields."""
    w = s.reshape(-1, SCALE_WORDS)[0].cpu()
    f = w.view(torch.float32)
    return {"amax": float(f[0]), "bias": int(w[1]), "scale": float(f[2]),
            "scale_inv": float(f[3]), "flags": int(w[4]) & 0xFFFFFFFF,
            "reduce_bits": int(w[5]) & 0xFFFFFFFF, "sat_count": int(w[7]) & 0xFFFFFFFF,
            "gen_max": (int(w[8]) & 0xFFFFFFFF) | ((int(w[9]) & 0xFFFFFFFF) << 32),
            "epoch": (int(w[10]) & 0xFFFFFFFF) | ((int(w[11]) & 0xFFFFFFFF) << 32)}


def fp8_scale_reset(s: torch.Tensor) -> None:
    n = s.numel() // SCALE_WORDS
    check(load().fp8_scale_reset(_dev(s, torch.int32, "s"), n, _stream(s)), "fp8_scale_reset")


def fp8_amax(x: torch.Tensor, s: torch.Tensor) -> None:
    check(load().fp8_amax(_dev(x, torch.bfloat16, "x"), x.numel(), _dev(s, torch.int32, "s"),
                          _stream(x)), "fp8_amax")


def fp8_scale(fmt, s: torch.Tensor, margin: int = 0, mu_log2: int = 0) -> None:
    check(load().fp8_scale(_fmt(fmt), margin, mu_log2, _dev(s, torch.int32, "s"), _stream(s)),
          "fp8_scale")


def fp8_amax_scale(x: torch.Tensor, fmt, s: torch.Tensor, margin: int = 0, mu_log2: int = 0) -> None:
    check(load().fp8_amax_scale(_dev(x, torch.bfloat16, "x"), x.numel(), _fmt(fmt), margin, mu_log2,
                                _dev(s, torch.int32, "s"), _stream(x)), "fp8_amax_scale")


def fp8_bias_host(amax: float, fmt, margin: int = 0, mu_log2: int = 0):
    flags = ctypes.c_uint32(0)
    b = load().fp8_bias_host(float(amax), _fmt(fmt), margin, mu_log2, ctypes.byref(flags))
    return int(b), int(flags.value)


def fp8_scale_fixed(s: torch.Tensor, bias: int) -> None:
    """FP8-CSCALE: set the record to a constant bias (scale 2^bias)."""
    check(load().fp8_scale_fixed(_dev(s, torch.int32, "s"), int(bias), _stream(s)), "fp8_scale_fixed")


def fp8_cast(x: torch.Tensor, fmt, s: torch.Tensor, out_row: Optional[torch.Tensor] = None,
             out_t: Optional[torch.Tensor] = None, rowwise: bool = True, transposed: bool = True):
    """Cast a bf16 [rows, cols] matrix; returns (rowwise [rows, cols] u8 or None,
    transposed [cols, rows] u8 or None)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    if rowwise and out_row is None:
        out_row = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if transposed and out_t is None:
        out_t = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    check(load().fp8_cast(_dev(x, torch.bfloat16, "x"), rows, cols, _fmt(fmt), _dev(s, torch.int32, "s"),
                          _dev(out_row, torch.uint8, "out_row"), _dev(out_t, torch.uint8, "out_t"),
                          _stream(x)), "fp8_cast")
    return out_row, out_t


def fp8_quantize(x: torch.Tensor, fmt, s: torch.Tensor, margin: int = 0, mu_log2: int = 0,
                 out_row: Optional[torch.Tensor] = None, out_t: Optional[torch.Tensor] = None,
                 rowwise: bool = True, transposed: bool = True):
    """amax + scale + cast (+ transpose) of a bf16 [rows, cols] matrix in one
    call; returns (rowwise or None, transposed or None)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    if rowwise and out_row is None:
        out_row = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if transposed and out_t is None:
        out_t = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    check(load().fp8_quantize(_dev(x, torch.bfloat16, "x"), rows, cols, _fmt(fmt), margin, mu_log2,
                              _dev(s, torch.int32, "s"), _dev(out_row, torch.uint8, "out_row"),
                              _dev(out_t, torch.uint8, "out_t"), _stream(x)), "fp8_quantize")
    return out_row, out_t


def fp8_quantize_spec(x: torch.Tensor, fmt, s: torch.Tensor, margin: int = 0, mu_log2: int = 0,
                      out_row: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp8_quantize (row-major output) in one pass that casts with the bias
    the record kept from its previous call, plus a check that recasts only
    if the tensor's own amax gives another bias. Same bytes and record."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    if out_row is None:
        out_row = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    check(load().fp8_quantize_spec(_dev(x, torch.bfloat16, "x"), rows, cols, _fmt(fmt), margin, mu_log2,
                                   _dev(s, torch.int32, "s"), _dev(out_row, torch.uint8, "out_row"), _stream(x)),
          "fp8_quantize_spec")
    return out_row


def fp8_quantize_batch(tensors):
    """fp8_quantize of up to 4 tensors in two launches (one amax pass over
    all, then all casts), each with its own record. tensors: list of dicts
    with fp8_quantize's keyword arguments (x, fmt, s, and optionally margin,
    mu_log2, out_row, out_t, rowwise, transposed). Returns a list of
    (rowwise or None, transposed or None)."""
    n = len(tensors)
    if not 1 <= n <= _lib.QUANTIZE_BATCH_MAX:
        raise ValueError(f"1 to {_lib.QUANTIZE_BATCH_MAX} tensors per batch")
    args = (QuantizeArgs * n)()
    outs = []
    for i, d in enumerate(tensors):
        x = d["x"]
        if x.dim() != 2:
            raise ValueError("x must be 2-D")
        rows, cols = x.shape
        out_row, out_t = d.get("out_row"), d.get("out_t")
        if d.get("rowwise", True) and out_row is None:
            out_row = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        if d.get("transposed", True) and out_t is None:
            out_t = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
        args[i] = QuantizeArgs(_dev(x, torch.bfloat16, "x"), rows, cols, _fmt(d["fmt"]), d.get("margin", 0),
                               d.get("mu_log2", 0), _dev(d["s"], torch.int32, "s"),
                               _dev(out_row, torch.uint8, "out_row"), _dev(out_t, torch.uint8, "out_t"))
        outs.append((out_row, out_t))
    check(load().fp8_quantize_batch(args, n, _stream(tensors[0]["x"])), "fp8_quantize_batch")
    return outs


def fp8_gemm_nt(a: torch.Tensor, fa, sa: torch.Tensor, b: torch.Tensor, fb, sb: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C[M, N] (bf16) = 2^-(bias_a + bias_b) * A[M, R] . B[N, R]^T on FP8 codes."""
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shape mismatch: A {tuple(a.shape)}, B {tuple(b.shape)}")
    M, R = a.shape
    N = b.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    check(load().fp8_gemm_nt(_dev(a, torch.uint8, "A"), _fmt(fa), _dev(sa, torch.int32, "sa"),
                             _dev(b, torch.uint8, "B"), _fmt(fb), _dev(sb, torch.int32, "sb"),
                             M, N, R, _dev(out, torch.bfloat16, "out"), _stream(a)), "fp8_gemm_nt")
    return out


LAYOUTS = {"rows": FP8_OPERAND_ROWS, "cols": FP8_OPERAND_COLS}


def _gemm_args(a: torch.Tensor, fa, sa: torch.Tensor, b: torch.Tensor, fb, sb: torch.Tensor,
               out: Optional[torch.Tensor], a_layout: str, b_layout: str):
    """Shape checks and the fp8_gemm argument set (as a GemmArgs struct)."""
    if a_layout not in LAYOUTS or b_layout not in LAYOUTS:
        raise ValueError("layouts are 'rows' or 'cols'")
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, Ra = (a.shape[1], a.shape[0]) if a_layout == "cols" else tuple(a.shape)
    N, Rb = (b.shape[1], b.shape[0]) if b_layout == "cols" else tuple(b.shape)
    if Ra != Rb:
        raise ValueError(f"reduction mismatch: A {tuple(a.shape)} ({a_layout}), B {tuple(b.shape)} ({b_layout})")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    args = GemmArgs(_dev(a, torch.uint8, "A"), _fmt(fa), LAYOUTS[a_layout], _dev(sa, torch.int32, "sa"),
                    _dev(b, torch.uint8, "B"), _fmt(fb), LAYOUTS[b_layout], _dev(sb, torch.int32, "sb"),
                    M, N, Ra, _dev(out, torch.bfloat16, "out"))
    return args, out


def fp8_gemm(a: torch.Tensor, fa, sa: torch.Tensor, b: torch.Tensor, fb, sb: torch.Tensor,
             out: Optional[torch.Tensor] = None, a_layout: str = "rows", b_layout: str = "rows",
             workspace: Optional[torch.Tensor] = None, split: str = "auto") -> torch.Tensor:
    """C[M, N] (bf16) = 2^-(bias_a + bias_b) * sum_r A(i, r) B(j, r) on FP8 codes,
    each operand either "rows" (A [M, R], B [N, R]) or "cols" (A [R, M], B [R, N]).
    With a workspace (uint8 device tensor, see gemm_workspace_bytes) the
    last partial wave of an E4M3 x E4M3 GEMM may be split (fp8_gemm_ws;
    split "auto", "never" or "tail")."""
    g, out = _gemm_args(a, fa, sa, b, fb, sb, out, a_layout, b_layout)
    if workspace is None:
        check(load().fp8_gemm(g.A, g.fa, g.la, g.sa, g.B, g.fb, g.lb, g.sb, g.M, g.N, g.R, g.C, _stream(a)),
              "fp8_gemm")
    else:
        check(load().fp8_gemm_ws(g.A, g.fa, g.la, g.sa, g.B, g.fb, g.lb, g.sb, g.M, g.N, g.R, g.C, SPLITS[split],
                                 _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(a)),
              "fp8_gemm_ws")
    return out


SPLITS = {"auto": FP8_SPLIT_AUTO, "never": FP8_SPLIT_NEVER, "tail": FP8_SPLIT_TAIL}


def fp8_gemm_noalloc(a: torch.Tensor, fa, sa: torch.Tensor, b: torch.Tensor, fb, sb: torch.Tensor,
                     out: torch.Tensor, a_layout: str = "rows", b_layout: str = "rows",
                     split: str = "auto") -> torch.Tensor:
    """fp8_gemm with a workspace, the split's partials in the library's own
    device scratch (fp8_gemm_noalloc): no device memory is allocated, so
    `out` is required. Calls that overlap on one GPU share that scratch."""
    if out is None:
        raise ValueError("fp8_gemm_noalloc needs the output tensor")
    g, out = _gemm_args(a, fa, sa, b, fb, sb, out, a_layout, b_layout)
    check(load().fp8_gemm_noalloc(g.A, g.fa, g.la, g.sa, g.B, g.fb, g.lb, g.sb, g.M, g.N, g.R, g.C, SPLITS[split],
                                  _stream(a)), "fp8_gemm_noalloc")
    return out


def gemm_workspace_bytes(fa, fb, M: int, N: int, R: int, split: str = "auto") -> int:
    """Workspace bytes fp8_gemm(..., workspace=, split=) uses for this GEMM
    on the current device (0: it would not split)."""
    return int(load().fp8_gemm_workspace_bytes(_fmt(fa), _fmt(fb), M, N, R, SPLITS[split]))


def fp8_gemm_pair(first: dict, second: dict):
    """Two fp8_gemm calls enqueued together (one launch for a linear's
    dgrad + wgrad pair); each dict holds fp8_gemm's keyword arguments
    (a, fa, sa, b, fb, sb, and optionally out, a_layout, b_layout). Returns
    the two outputs."""
    def one(d):
        return _gemm_args(d["a"], d["fa"], d["sa"], d["b"], d["fb"], d["sb"], d.get("out"),
                          d.get("a_layout", "rows"), d.get("b_layout", "rows"))
    g0, out0 = one(first)
    g1, out1 = one(second)
    check(load().fp8_gemm_pair(ctypes.byref(g0), ctypes.byref(g1), _stream(first["a"])), "fp8_gemm_pair")
    return out0, out1


class LinearWorkspace:
    """Device buffers of one FP8 linear: the row-major FP8 copies of X, W
    and dY, the three scaling records and, with transposed=True, the
    transposed FP8 copies as well (the linear entry points then also write
    them; their GEMMs never need them), and the forward GEMM's workspace
    when its shape splits the last wave."""

    def __init__(self, M: int, K: int, N: int, device="cuda", transposed: bool = False):
        u8 = dict(dtype=torch.uint8, device=device)
        self.M, self.K, self.N = M, K, N
        self.x8 = torch.empty((M, K), **u8)
        self.w8 = torch.empty((K, N), **u8)
        self.dy8 = torch.empty((M, N), **u8)
        self.x8t = torch.empty((K, M), **u8) if transposed else None
        self.w8t = torch.empty((N, K), **u8) if transposed else None
        self.dy8t = torch.empty((N, M), **u8) if transposed else None
        self.scales = new_scale(3, device)
        self.sx, self.sw, self.sdy = self.scales[0], self.scales[1], self.scales[2]
        # forward GEMM workspace (last-wave split), when this shape uses one
        nb = int(load().fp8_linear_scratch_bytes(M, K, N)) if torch.device(device).type == "cuda" else 0
        self.scratch = torch.empty(nb, **u8) if nb else None
        self.c = LinearWs(*[None if t is None else t.data_ptr()
                            for t in (self.x8, self.x8t, self.w8, self.w8t, self.dy8, self.dy8t, self.sx,
                                      self.sw, self.sdy, self.scratch)], nb)


def fp8_linear_fwd(X: torch.Tensor, W: torch.Tensor, ws: LinearWorkspace, margin: int = 0,
                   Y: Optional[torch.Tensor] = None) -> torch.Tensor:
    M, K = X.shape
    K2, N = W.shape
    if K2 != K or (ws.M, ws.K, ws.N) != (M, K, N):
        raise ValueError("shape mismatch between X, W and the workspace")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    check(load().fp8_linear_fwd(_dev(X, torch.bfloat16, "X"), _dev(W, torch.bfloat16, "W"), M, K, N,
                                margin, ctypes.byref(ws.c), _dev(Y, torch.bfloat16, "Y"), _stream(X)),
          "fp8_linear_fwd")
    return Y


def fp8_linear_bwd(dY: torch.Tensor, ws: LinearWorkspace, margin: int = 0, mu_log2: int = 0,
                   dX: Optional[torch.Tensor] = None, dW: Optional[torch.Tensor] = None,
                   need_dx: bool = True, need_dw: bool = True):
    M, K, N = ws.M, ws.K, ws.N
    if tuple(dY.shape) != (M, N):
        raise ValueError("dY has the wrong shape")
    if need_dx and dX is None:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=dY.device)
    if need_dw and dW is None:
        dW = torch.empty((K, N), dtype=torch.bfloat16, device=dY.device)
    check(load().fp8_linear_bwd(_dev(dY, torch.bfloat16, "dY"), M, K, N, margin, mu_log2,
                                ctypes.byref(ws.c), _dev(dX, torch.bfloat16, "dX"),
                                _dev(dW, torch.bfloat16, "dW"), _stream(dY)), "fp8_linear_bwd")
    return dX, dW


# Workspaces of the autograd path, reused across calls: free ones per
# (M, K, N, device). A forward takes one (or builds one when none is free)
# and holds it through a lease kept in the autograd context, since its FP8
# copies and records are the backward's inputs; the lease gives it back
# when the context is freed (after the backward, or when the graph is
# dropped), so a training loop settles on one or two workspaces per shape
# and allocates nothing more. Reuse is ordered by the stream: callers that
# run forward and backward on different streams must order them.
_WS_POOL = {}
_WS_POOL_KEEP = 4            # free workspaces kept per shape


class _Lease:
    __slots__ = ("key", "ws")

    def __init__(self, key, ws):
        self.key, self.ws = key, ws

    def __del__(self):
        try:
            free = _WS_POOL.setdefault(self.key, [])
            if len(free) < _WS_POOL_KEEP:
                free.append(self.ws)
        except Exception:     # interpreter shutdown: the pool may be gone
            pass


def _lease_workspace(M: int, K: int, N: int, device) -> _Lease:
    key = (M, K, N, str(torch.device(device)))
    free = _WS_POOL.get(key)
    ws = free.pop() if free else LinearWorkspace(M, K, N, device)
    return _Lease(key, ws)


def release_workspaces() -> None:
    """Drop the free workspaces the autograd path keeps for reuse."""
    _WS_POOL.clear()


class _FP8LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, X, W, margin, mu_log2):
        Xc, Wc = X.contiguous(), W.contiguous()
        lead = Xc.shape[:-1]
        X2 = Xc.reshape(-1, Xc.shape[-1])
        lease = _lease_workspace(X2.shape[0], X2.shape[1], Wc.shape[1], X.device)
        Y = fp8_linear_fwd(X2, Wc, lease.ws, margin)
        ctx.lease, ctx.margin, ctx.mu_log2, ctx.lead = lease, margin, mu_log2, lead
        return Y.reshape(*lead, Wc.shape[1])

    @staticmethod
    def backward(ctx, dY):
        dY2 = dY.contiguous().reshape(-1, dY.shape[-1])
        if dY2.dtype != torch.bfloat16:
            dY2 = dY2.to(torch.bfloat16)
        dX, dW = fp8_linear_bwd(dY2, ctx.lease.ws, ctx.margin, ctx.mu_log2,
                                need_dx=ctx.needs_input_grad[0], need_dw=ctx.needs_input_grad[1])
        if dX is not None:
            dX = dX.reshape(*ctx.lead, dX.shape[-1])
        return dX, dW, None, None


def linear(X: torch.Tensor, W: torch.Tensor, margin: int = 0, mu_log2: int = 0) -> torch.Tensor:
    """Y = X W with per-tensor dynamically scaled FP8 (E4M3 X and W, E5M2 dY).
    X [..., K] bf16, W [K, N] bf16 (in x out)."""
    return _FP8LinearFn.apply(X, W, margin, mu_log2)


class Linear(torch.nn.Module):
    """Drop-in FP8 linear layer (no bias term); weight stored [in, out] in bf16."""

    def __init__(self, in_features: int, out_features: int, margin: int = 0, mu_log2: int = 0,
                 device=None):
        super().__init__()
        self.weight = torch.nn.Parameter(
            torch.empty((in_features, out_features), dtype=torch.bfloat16, device=device))
        torch.nn.init.normal_(self.weight, std=0.02)
        self.margin, self.mu_log2 = margin, mu_log2

    def forward(self, x):
        return linear(x, self.weight, self.margin, self.mu_log2)


def fp8_wgrad_fp8(x8: torch.Tensor, sx: torch.Tensor, dy8: torch.Tensor, sdy: torch.Tensor,
                  margin: int = 0, mu_log2: int = 0, dW: Optional[torch.Tensor] = None,
                  s_dw: Optional[torch.Tensor] = None, dw8: Optional[torch.Tensor] = None,
                  dw8t: Optional[torch.Tensor] = None, transposed: bool = False, x_layout: str = "rows",
                  dy_layout: str = "rows"):
    """FP8 weight gradient: dW = X^T dY (bf16, the GEMM's epilogue also
    takes max |dW|), then dW in E5M2 with the bias from that amax, the margin
    and mu = 2^mu_log2. x8: X^T [K, M] ("rows") or X [M, K] ("cols"); dy8:
    dY^T [N, M] ("rows") or dY [M, N] ("cols"). Returns (dW [K, N] bf16,
    dw8 [K, N] u8, dw8t [N, K] u8 or None, s_dw)."""
    if x_layout not in LAYOUTS or dy_layout not in LAYOUTS:
        raise ValueError("layouts are 'rows' or 'cols'")
    if x8.dim() != 2 or dy8.dim() != 2:
        raise ValueError("x8 and dy8 must be 2-D")
    K, M = (x8.shape[1], x8.shape[0]) if x_layout == "cols" else tuple(x8.shape)
    N, M2 = (dy8.shape[1], dy8.shape[0]) if dy_layout == "cols" else tuple(dy8.shape)
    if M != M2:
        raise ValueError(f"shape mismatch: x8 {tuple(x8.shape)} ({x_layout}), dy8 {tuple(dy8.shape)} ({dy_layout})")
    dev = x8.device
    if dW is None:
        dW = torch.empty((K, N), dtype=torch.bfloat16, device=dev)
    if dw8 is None:
        dw8 = torch.empty((K, N), dtype=torch.uint8, device=dev)
    if transposed and dw8t is None:
        dw8t = torch.empty((N, K), dtype=torch.uint8, device=dev)
    if s_dw is None:
        s_dw = new_scale(1, dev)[0]
    check(load().fp8_wgrad_fp8(_dev(x8, torch.uint8, "x8"), LAYOUTS[x_layout], _dev(sx, torch.int32, "sx"),
                               _dev(dy8, torch.uint8, "dy8"), LAYOUTS[dy_layout], _dev(sdy, torch.int32, "sdy"),
                               K, N, M, margin, mu_log2, _dev(dW, torch.bfloat16, "dW"),
                               _dev(s_dw, torch.int32, "s_dw"), _dev(dw8, torch.uint8, "dw8"),
                               _dev(dw8t, torch.uint8, "dw8t"), _stream(x8)), "fp8_wgrad_fp8")
    return dW, dw8, dw8t, s_dw


def prepare_weight(W: torch.Tensor, margin: int = 0, fixed_bias: Optional[int] = None, layout: str = "cols"):
    """Cast a bf16 weight W [K, N] once for inference (post-training
    quantisation): returns (w8, record sw) with w8 the E4M3 codes, row-major
    [K, N] for layout "cols" (read reduction-major by the forward GEMM, as in
    training; the faster layout) or transposed [N, K] for "rows". The bias
    comes from amax(W) and the margin, or is fixed_bias (FP8-CSCALE)."""
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    if layout not in LAYOUTS:
        raise ValueError("layout is 'rows' or 'cols'")
    sw = new_scale(1, W.device)[0]
    if fixed_bias is None:
        fp8_amax_scale(W, "e4m3", sw, margin)
    else:
        fp8_scale_fixed(sw, fixed_bias)
    w8, w8t = fp8_cast(W, "e4m3", sw, rowwise=layout == "cols", transposed=layout == "rows")
    return (w8 if layout == "cols" else w8t), sw


def fp8_linear_fwd_cached(X: torch.Tensor, w8: torch.Tensor, sw: torch.Tensor, x8: torch.Tensor,
                          sx: torch.Tensor, margin: int = 0, x_scaling: str = "amax",
                          Y: Optional[torch.Tensor] = None, w_layout: str = "cols") -> torch.Tensor:
    """Y [M, N] = X [M, K] W from a prepared FP8 weight and its record sw:
    w8 [K, N] (w_layout "cols", prepare_weight's default) or [N, K] ("rows").
    x_scaling "amax": X's bias from amax(X) and the margin (written to sx);
    "fixed": the bias already in sx (fp8_scale_fixed)."""
    if w_layout not in LAYOUTS:
        raise ValueError("w_layout is 'rows' or 'cols'")
    if X.dim() != 2 or w8.dim() != 2:
        raise ValueError("X and w8 must be 2-D")
    M, K = X.shape
    Kw, N = (w8.shape[0], w8.shape[1]) if w_layout == "cols" else (w8.shape[1], w8.shape[0])
    if Kw != K:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, w8 {tuple(w8.shape)} ({w_layout})")
    if tuple(x8.shape) != (M, K):
        raise ValueError("x8 must be [M, K]")
    try:
        mode = SCALINGS[x_scaling]
    except KeyError:
        raise ValueError(f"unknown x_scaling {x_scaling!r}") from None
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    check(load().fp8_linear_fwd_cached(_dev(X, torch.bfloat16, "X"), M, K, N, margin, mode,
                                       _dev(w8, torch.uint8, "w8"), LAYOUTS[w_layout], _dev(sw, torch.int32, "sw"),
                                       _dev(x8, torch.uint8, "x8"), _dev(sx, torch.int32, "sx"),
                                       _dev(Y, torch.bfloat16, "Y"), _stream(X)), "fp8_linear_fwd_cached")
    return Y


class InferenceLinear(torch.nn.Module):
    """Forward-only FP8 linear on a weight cast once (post-training
    quantisation). X is scaled from its amax per call, or with a fixed bias
    (FP8-CSCALE) when x_fixed_bias is given."""

    def __init__(self, W: torch.Tensor, margin: int = 0, w_fixed_bias: Optional[int] = None,
                 x_fixed_bias: Optional[int] = None):
        super().__init__()
        self.margin = margin
        self.w8, self.sw = prepare_weight(W, margin, w_fixed_bias)
        self.sx = new_scale(1, W.device)[0]
        self.x_scaling = "amax"
        if x_fixed_bias is not None:
            fp8_scale_fixed(self.sx, x_fixed_bias)
            self.x_scaling = "fixed"
        self._x8 = None

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        shape = x.shape
        x2 = x.reshape(-1, shape[-1]).contiguous()
        if self._x8 is None or tuple(self._x8.shape) != tuple(x2.shape):
            self._x8 = torch.empty(x2.shape, dtype=torch.uint8, device=x2.device)
        y = fp8_linear_fwd_cached(x2, self.w8, self.sw, self._x8, self.sx, self.margin, self.x_scaling)
        return y.reshape(*shape[:-1], y.shape[-1])


class AdamState:
    """O2 optimizer state of one weight tensor of n elements: first moment
    m1 (E4M3 codes), second moment m2 and master weights w16 (FP16 bits),
    each with its scaling record (s_m1, s_m2, s_w)."""

    def __init__(self, W: torch.Tensor):
        if W.dtype != torch.bfloat16 or not W.is_cuda:
            raise ValueError("W must be a bf16 device tensor")
        self.shape = tuple(W.shape)
        self.n = W.numel()
        dev = W.device
        self.m1 = torch.zeros(self.n, dtype=torch.uint8, device=dev)
        self.m2 = torch.zeros(self.n, dtype=torch.int16, device=dev)
        self.w16 = torch.empty(self.n, dtype=torch.int16, device=dev)
        self.scales = new_scale(3, dev)
        self.s_m1, self.s_m2, self.s_w = self.scales[0], self.scales[1], self.scales[2]
        self.step_count = 0
        self.alt = None     # second buffer set of fp8_adam_step_spec (out of place), made on first use
        fp8_adam_init_master(W.reshape(-1).contiguous(), self.w16, self.s_w)


def fp8_adam_init_master(w_bf16: torch.Tensor, w16: torch.Tensor, s_w: torch.Tensor) -> None:
    check(load().fp8_adam_init_master(w_bf16.numel(), _dev(w_bf16, torch.bfloat16, "w_bf16"),
                                      _dev(w16, torch.int16, "w16"), _dev(s_w, torch.int32, "s_w"),
                                      _stream(w_bf16)), "fp8_adam_init_master")


def fp8_adam_step(state: AdamState, g8: torch.Tensor, s_g: torch.Tensor, lr: float, beta1: float = 0.9,
                  beta2: float = 0.95, eps: float = 1e-8, weight_decay: float = 0.0,
                  w_bf16: Optional[torch.Tensor] = None, step: Optional[int] = None) -> Optional[torch.Tensor]:
    """One O2 Adam step on `state` with the E5M2 gradient g8 (n codes, any
    shape) and its record s_g; writes the new bf16 weights to w_bf16 if
    given. `step` defaults to the state's own count + 1."""
    if g8.numel() != state.n:
        raise ValueError("gradient size differs from the state's")
    t = state.step_count + 1 if step is None else int(step)
    check(load().fp8_adam_step(state.n, _dev(g8, torch.uint8, "g8"), _dev(s_g, torch.int32, "s_g"),
                               _dev(state.m1, torch.uint8, "m1"), _dev(state.s_m1, torch.int32, "s_m1"),
                               _dev(state.m2, torch.int16, "m2"), _dev(state.s_m2, torch.int32, "s_m2"),
                               _dev(state.w16, torch.int16, "w16"), _dev(state.s_w, torch.int32, "s_w"),
                               _dev(w_bf16, torch.bfloat16, "w_bf16"), lr, beta1, beta2, eps, weight_decay, t,
                               _stream(g8)), "fp8_adam_step")
    state.step_count = t
    return w_bf16


def fp8_adam_step_spec(state: AdamState, g8: torch.Tensor, s_g: torch.Tensor, lr: float, beta1: float = 0.9,
                       beta2: float = 0.95, eps: float = 1e-8, weight_decay: float = 0.0,
                       w_bf16: Optional[torch.Tensor] = None, step: Optional[int] = None,
                       missed: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """fp8_adam_step's step in one pass over the state when no scale changes
    (fp8_adam_step_spec): the new state goes to the state's second buffer
    set (made on first use), which then becomes the current one. missed: an
    optional device int32 tensor of one element that receives the bit mask
    of the records whose scale changed (bit 0 m1, 1 m2, 2 w)."""
    if g8.numel() != state.n:
        raise ValueError("gradient size differs from the state's")
    if missed is not None and (missed.numel() < 1 or missed.dtype != torch.int32):
        raise ValueError("missed must be an int32 tensor of at least one element")
    t = state.step_count + 1 if step is None else int(step)
    if state.alt is None:
        state.alt = (torch.empty_like(state.m1), torch.empty_like(state.m2), torch.empty_like(state.w16))
    m1o, m2o, w16o = state.alt
    check(load().fp8_adam_step_spec(state.n, _dev(g8, torch.uint8, "g8"), _dev(s_g, torch.int32, "s_g"),
                                    _dev(state.m1, torch.uint8, "m1"), _dev(state.m2, torch.int16, "m2"),
                                    _dev(state.w16, torch.int16, "w16"), _dev(m1o, torch.uint8, "m1_out"),
                                    _dev(m2o, torch.int16, "m2_out"), _dev(w16o, torch.int16, "w16_out"),
                                    _dev(state.s_m1, torch.int32, "s_m1"), _dev(state.s_m2, torch.int32, "s_m2"),
                                    _dev(state.s_w, torch.int32, "s_w"), _dev(w_bf16, torch.bfloat16, "w_bf16"),
                                    _dev(missed, torch.int32, "missed"), lr, beta1, beta2, eps, weight_decay, t,
                                    _stream(g8)), "fp8_adam_step_spec")
    state.alt = (state.m1, state.m2, state.w16)
    state.m1, state.m2, state.w16 = m1o, m2o, w16o
    state.step_count = t
    return w_bf16
