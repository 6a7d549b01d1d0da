"""ctypes loader for libfp8lin.so (the C ABI declared in include/fp8lin.h).

Loading fails loudly: there is no CPU fallback for any entry point."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FP8LIN_LIB", os.path.join(_HERE, "lib", "libfp8lin.so"))

c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_vp = ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/fp8lin.h
SIGNATURES = {
    "fp8_status_str": (ctypes.c_char_p, [c_int]),
    "fp8_abi_version": (c_int, []),
    "fp8_scale_reset": (c_int, [c_vp, c_i64, c_vp]),
    "fp8_amax": (c_int, [c_vp, c_i64, c_vp, c_vp]),
    "fp8_scale": (c_int, [c_int, c_int, c_int, c_vp, c_vp]),
    "fp8_amax_scale": (c_int, [c_vp, c_i64, c_int, c_int, c_int, c_vp, c_vp]),
    "fp8_bias_host": (ctypes.c_int32, [ctypes.c_float, c_int, c_int, c_int, ctypes.POINTER(ctypes.c_uint32)]),
    "fp8_quantize": (c_int, [c_vp, c_i64, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp]),
    "fp8_quantize_batch": (c_int, [c_vp, c_int, c_vp]),
    "fp8_quantize_spec": (c_int, [c_vp, c_i64, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_vp]),
    "fp8_scale_fixed": (c_int, [c_vp, ctypes.c_int32, c_vp]),
    "fp8_cast": (c_int, [c_vp, c_i64, c_i64, c_int, c_vp, c_vp, c_vp, c_vp]),
    "fp8_gemm_nt": (c_int, [c_vp, c_int, c_vp, c_vp, c_int, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]),
    "fp8_gemm": (c_int, [c_vp, c_int, c_int, c_vp, c_vp, c_int, c_int, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]),
    "fp8_gemm_pair": (c_int, [c_vp, c_vp, c_vp]),
    "fp8_gemm_ws": (c_int, [c_vp, c_int, c_int, c_vp, c_vp, c_int, c_int, c_vp, c_i64, c_i64, c_i64, c_vp, c_int,
                            c_vp, ctypes.c_size_t, c_vp]),
    "fp8_gemm_noalloc": (c_int, [c_vp, c_int, c_int, c_vp, c_vp, c_int, c_int, c_vp, c_i64, c_i64, c_i64, c_vp,
                                 c_int, c_vp]),
    "fp8_gemm_workspace_bytes": (ctypes.c_size_t, [c_int, c_int, c_i64, c_i64, c_i64, c_int]),
    "fp8_linear_scratch_bytes": (ctypes.c_size_t, [c_i64, c_i64, c_i64]),
    "fp8_linear_fwd": (c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_int, c_vp, c_vp, c_vp]),
    "fp8_linear_bwd": (c_int, [c_vp, c_i64, c_i64, c_i64, c_int, c_int, c_vp, c_vp, c_vp, c_vp]),
    "fp8_linear_fwd_cached": (c_int, [c_vp, c_i64, c_i64, c_i64, c_int, c_int, c_vp, c_int, c_vp, c_vp, c_vp,
                                      c_vp, c_vp]),
    "fp8_wgrad_fp8": (c_int, [c_vp, c_int, c_vp, c_vp, c_int, c_vp, c_i64, c_i64, c_i64, c_int, c_int, c_vp, c_vp,
                              c_vp, c_vp, c_vp]),
    "fp8_adam_init_master": (c_int, [c_i64, c_vp, c_vp, c_vp, c_vp]),
    "fp8_adam_step": (c_int, [c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_float,
                              ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_int32, c_vp]),
    "fp8_adam_step_spec": (c_int, [c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                   c_vp, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                   ctypes.c_float, ctypes.c_int32, c_vp]),
}

FP8_E4M3, FP8_E5M2 = 0, 1
FP8_OPERAND_ROWS, FP8_OPERAND_COLS = 0, 1
FP8_OK, FP8_ERR_INVALID, FP8_ERR_UNSUPPORTED, FP8_ERR_HIP = 0, 1, 2, 3
FLAG_NONFINITE, FLAG_ZERO, FLAG_CLAMPED = 1, 2, 4
FP8_SCALING_AMAX, FP8_SCALING_FIXED = 0, 1
FP8_SPLIT_AUTO, FP8_SPLIT_NEVER, FP8_SPLIT_TAIL = 0, 1, 2
ABI_VERSION = 13
FP8_NOALLOC_SCRATCH_BYTES = 128 * 2 * 65536 * 4   # the device scratch of fp8_gemm_noalloc


class LinearWs(ctypes.Structure):
    """fp8_linear_ws: host struct of device pointers."""
    _fields_ = [("x8", c_vp), ("x8t", c_vp), ("w8", c_vp), ("w8t", c_vp), ("dy8", c_vp),
                ("dy8t", c_vp), ("sx", c_vp), ("sw", c_vp), ("sdy", c_vp), ("scratch", c_vp),
                ("scratch_bytes", ctypes.c_size_t)]


class QuantizeArgs(ctypes.Structure):
    """fp8_quantize_args: the arguments of one fp8_quantize call (host struct)."""
    _fields_ = [("x", c_vp), ("rows", c_i64), ("cols", c_i64), ("fmt", c_int), ("margin", c_int),
                ("mu_log2", c_int), ("s", c_vp), ("out_rowwise", c_vp), ("out_transposed", c_vp)]


QUANTIZE_BATCH_MAX = 4


class GemmArgs(ctypes.Structure):
    """fp8_gemm_args: the arguments of one fp8_gemm call (host struct)."""
    _fields_ = [("A", c_vp), ("fa", c_int), ("la", c_int), ("sa", c_vp), ("B", c_vp), ("fb", c_int),
                ("lb", c_int), ("sb", c_vp), ("M", c_i64), ("N", c_i64), ("R", c_i64), ("C", c_vp)]


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libfp8lin.so not found at {LIB_PATH}; build it with "
            "`python -m tensor_scaled_fp8_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.fp8_abi_version() != ABI_VERSION:
        raise ImportError(f"libfp8lin ABI {lib.fp8_abi_version()} != expected {ABI_VERSION}")
    _lib = lib
    return lib


def check(status: int, what: str) -> None:
    if status != FP8_OK:
        msg = load().fp8_status_str(status).decode()
        raise RuntimeError(f"{what}: {msg} (status {status})")
