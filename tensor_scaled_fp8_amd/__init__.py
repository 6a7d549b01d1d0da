"""Per-tensor dynamically scaled FP8 linear layer for MI355X (gfx950).

The computation runs in hand-written HIP kernels behind a C ABI
(include/fp8lin.h, libfp8lin.so); this package is its Python binding."""
from ._lib import (FLAG_CLAMPED, FLAG_NONFINITE, FLAG_ZERO, FP8_E4M3, FP8_E5M2, FP8_NOALLOC_SCRATCH_BYTES, LIB_PATH,
                   SIGNATURES, load)
from .binding import (AdamState, InferenceLinear, Linear, LinearWorkspace, fp8_amax, fp8_amax_scale,
                      fp8_bias_host, fp8_cast, fp8_gemm, fp8_gemm_noalloc, fp8_gemm_nt, fp8_gemm_pair, fp8_linear_bwd, gemm_workspace_bytes, fp8_linear_fwd,
                      fp8_linear_fwd_cached, fp8_quantize, fp8_quantize_batch, fp8_quantize_spec, fp8_scale, fp8_scale_fixed, fp8_scale_reset,
                      fp8_wgrad_fp8, fp8_adam_init_master, fp8_adam_step, fp8_adam_step_spec, linear, new_scale,
                      prepare_weight, read_scale, release_workspaces)
from .mu import MuScaler

__all__ = [
    "FLAG_CLAMPED", "FLAG_NONFINITE", "FLAG_ZERO", "FP8_E4M3", "FP8_E5M2", "FP8_NOALLOC_SCRATCH_BYTES", "LIB_PATH", "SIGNATURES",
    "load", "AdamState", "fp8_adam_init_master", "fp8_adam_step", "fp8_adam_step_spec", "InferenceLinear", "Linear", "LinearWorkspace", "fp8_amax", "fp8_amax_scale", "fp8_bias_host",
    "fp8_cast", "fp8_gemm", "fp8_gemm_noalloc", "fp8_gemm_nt", "fp8_gemm_pair", "gemm_workspace_bytes", "fp8_linear_bwd", "fp8_linear_fwd", "fp8_linear_fwd_cached", "fp8_quantize", "fp8_quantize_batch", "fp8_quantize_spec",
    "fp8_scale", "fp8_scale_fixed", "fp8_scale_reset", "fp8_wgrad_fp8", "linear", "MuScaler", "new_scale",
    "prepare_weight", "read_scale", "release_workspaces",
]
