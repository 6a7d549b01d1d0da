"""One FP8 linear, forward and backward, composed from the oracle steps.

[AMAX] "Proposed method", bullets 1-4: per-tensor amax and bias for X and W
(E4 format) and dY (E5 format), scale and cast, FP8 matmul, undo the scales.
[FP8LM] "Proposed method", O1, Eq. 3: mu scales the gradient (dY) only.

Layouts: X [M,K], W [K,N], dY [M,N], all row-major bf16 bit patterns.
"""
from __future__ import annotations

from .formats import E4M3, E5M2
from .gemm import gemm_nt
from .scaling import cast, scale_record


def linear_fwd_bwd(x_bits, w_bits, dy_bits, margin: int = 0, mu_log2: int = 0,
                   with_tolerance: bool = True, gemms: bool = True) -> dict:
    sx = scale_record(x_bits, E4M3, margin, 0)
    sw = scale_record(w_bits, E4M3, margin, 0)
    sdy = scale_record(dy_bits, E5M2, margin, mu_log2)
    x8, x8t = cast(x_bits, E4M3, sx["bias"])
    w8, w8t = cast(w_bits, E4M3, sw["bias"])
    dy8, dy8t = cast(dy_bits, E5M2, sdy["bias"])
    out = {"sx": sx, "sw": sw, "sdy": sdy, "x8": x8, "x8t": x8t, "w8": w8, "w8t": w8t,
           "dy8": dy8, "dy8t": dy8t}
    if gemms:
        out["Y"] = gemm_nt(x8, E4M3, sx["bias"], w8t, E4M3, sw["bias"], with_tolerance)
        out["dX"] = gemm_nt(dy8, E5M2, sdy["bias"], w8, E4M3, sw["bias"], with_tolerance)
        out["dW"] = gemm_nt(x8t, E4M3, sx["bias"], dy8t, E5M2, sdy["bias"], with_tolerance)
    return out
