"""Oracle: a plain, slow, CPU-only definition of the per-tensor dynamically
scaled FP8 linear layer (amax -> scale choice -> FP8 cast -> FP8 GEMMs).

TEST INFRASTRUCTURE ONLY. The package `tensor_scaled_fp8_amd` (the product)
never imports it; only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import or call it. It shares no code
with the HIP path: no kernels, headers, tables or helpers. The only common
code is `workloads`, which draws the seeded inputs and holds none of the
method's arithmetic.

Sources (cited by page title and section):
  [AMAX]  review of Perez, Zhang et al., "Training and inference of large
          language models using 8-bit floating point" (nubint.ai, Korean),
          section "Proposed method" (제안 방법), bullets 1-6.
  [FP8LM] reading note on Peng et al., "FP8-LM: Training FP8 Large Language
          Models" (notes.yuuk.io, Japanese), section "Proposed method"
          (提案手法), O1 optimisation, Eq. 3.

Readings where the pages are silent (each one is listed with its pin in the
design notes): OCP E4M3FN / E5M2 encodings with maxima 448 / 57344;
round-to-nearest-even with saturation; the bias is the floor of
log2(fmt_max / amax) minus the margin, plus log2(mu) for gradients, clamped
to [-126, 126]; the scale is 2^bias; outputs are bf16 rounded once to
nearest even.

Parity status: every function here is pinned by the `-m "not gpu"` tests in
tests/test_oracle_*.py, the compositions too: linear_fwd_bwd's routing of
the margin (all three tensors) and of mu (dY only) in test_oracle_linear.py,
adam.adam_step against a hand-written scalar AdamW with field-level decode,
closed-form biases and brute-force encoders in test_oracle_adam.py. The mu
update policy is not defined by the pages and is not implemented here (mu
is an input).
"""
from .formats import E4M3, E5M2, FORMATS, Fp8Format, decode_code, decode_table, encode
from .bf16 import bf16_to_f64, f64_to_bf16_rne, bf16_ulp
from .scaling import (FLAG_NONFINITE, FLAG_ZERO, FLAG_CLAMPED, BIAS_MIN, BIAS_MAX,
                      amax, compute_bias, scale_record, fixed_record, saturated_count, cast)
from .gemm import gemm_nt, gemm_nt_exact, gemm_nt_rows, tolerance
from .linear import linear_fwd_bwd
from . import adam

__all__ = [
    "E4M3", "E5M2", "FORMATS", "Fp8Format", "decode_code", "decode_table", "encode",
    "bf16_to_f64", "f64_to_bf16_rne", "bf16_ulp",
    "FLAG_NONFINITE", "FLAG_ZERO", "FLAG_CLAMPED", "BIAS_MIN", "BIAS_MAX",
    "amax", "compute_bias", "scale_record", "cast",
    "gemm_nt", "gemm_nt_exact", "gemm_nt_rows", "tolerance", "linear_fwd_bwd",
]
