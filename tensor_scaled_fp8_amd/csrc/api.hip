// C-ABI entry points of libfp8lin.so: argument validation, then kernel
// launches on the caller's stream. No allocation, no host synchronisation.
#include <string.h>

#include <cmath>

#include "fp8lin_internal.h"

using namespace fp8lin;

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool fmt_ok(int f) { return f == FP8_E4M3 || f == FP8_E5M2; }
inline bool int_ok(int v) { return v >= -kIntArgLimit && v <= kIntArgLimit; }
constexpr int64_t kMaxDim = (int64_t)1 << 31;  // per-dimension limit (tile indices are 32-bit)
inline fp8_status hip_status(hipError_t e) { return e == hipSuccess ? FP8_OK : FP8_ERR_HIP; }
// GEMM operands are addressed with 32-bit byte offsets
constexpr int64_t kMaxOperandBytes = (int64_t)1 << 32;
inline bool gemm_fits(int64_t M, int64_t N, int64_t R) {
  return M * R < kMaxOperandBytes && N * R < kMaxOperandBytes;
}

inline bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// the checks fp8_adam_step and fp8_adam_step_spec share; fills h
fp8_status adam_check(int64_t n, const uint8_t* g8, const fp8_scale_t* s_g, const void* m1, const fp8_scale_t* s_m1,
                      const void* m2, const fp8_scale_t* s_m2, const void* w16, const fp8_scale_t* s_w,
                      const void* w_bf16, float lr, float beta1, float beta2, float eps, float weight_decay,
                      int32_t step, AdamHyper& h) {
  if (n < 0 || step < 1) return FP8_ERR_INVALID;
  const fp8_scale_t* recs[] = {s_g, s_m1, s_m2, s_w};
  for (const fp8_scale_t* r : recs)
    if (!r || !aligned16(r)) return FP8_ERR_INVALID;
  if (!std::isfinite(lr) || !std::isfinite(eps) || !(eps > 0.0f) || !std::isfinite(weight_decay) ||
      !(weight_decay >= 0.0f) || !(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
    return FP8_ERR_INVALID;
  if (n % 16) return FP8_ERR_UNSUPPORTED;
  if (n > 0) {
    const void* p[] = {g8, m1, m2, w16};
    for (const void* q : p)
      if (!q || !aligned16(q)) return FP8_ERR_INVALID;
    if (w_bf16 && !aligned16(w_bf16)) return FP8_ERR_INVALID;
  }
  h.lr = lr;
  h.beta1 = beta1;
  h.beta2 = beta2;
  h.eps = eps;
  h.weight_decay = weight_decay;
  h.bc1 = (float)(1.0 / (1.0 - std::pow((double)beta1, (double)step)));
  h.bc2 = (float)(1.0 / (1.0 - std::pow((double)beta2, (double)step)));
  return FP8_OK;
}

// a device byte range; two ranges overlap when both are non-empty and meet
struct Range {
  const void* p;
  size_t bytes;
};
inline bool overlaps(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

}  // namespace

extern "C" {

const char* fp8_status_str(fp8_status s) {
  switch (s) {
    case FP8_OK: return "ok";
    case FP8_ERR_INVALID: return "invalid argument";
    case FP8_ERR_UNSUPPORTED: return "unsupported shape or format";
    case FP8_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

int fp8_abi_version(void) { return FP8LIN_ABI_VERSION; }

fp8_status fp8_scale_reset(fp8_scale_t* s_dev, int64_t count, hipStream_t stream) {
  if (count < 0 || (count > 0 && (!s_dev || !aligned16(s_dev)))) return FP8_ERR_INVALID;
  return hip_status(launch_scale_reset(s_dev, count, stream));
}

fp8_status fp8_amax(const void* x_bf16, int64_t n, fp8_scale_t* s_dev, hipStream_t stream) {
  if (n < 0 || !s_dev || !aligned16(s_dev)) return FP8_ERR_INVALID;
  if (n > 0 && (!x_bf16 || !aligned16(x_bf16))) return FP8_ERR_INVALID;
  return hip_status(launch_amax(x_bf16, n, s_dev, false, 0, 0, 0, stream));
}

fp8_status fp8_scale(fp8_fmt fmt, int margin, int mu_log2, fp8_scale_t* s_dev, hipStream_t stream) {
  if (!fmt_ok(fmt) || !int_ok(margin) || !int_ok(mu_log2) || !s_dev || !aligned16(s_dev))
    return FP8_ERR_INVALID;
  return hip_status(launch_scale(s_dev, fmt, margin, mu_log2, stream));
}

fp8_status fp8_amax_scale(const void* x_bf16, int64_t n, fp8_fmt fmt, int margin, int mu_log2,
                          fp8_scale_t* s_dev, hipStream_t stream) {
  if (n < 0 || !fmt_ok(fmt) || !int_ok(margin) || !int_ok(mu_log2) || !s_dev || !aligned16(s_dev))
    return FP8_ERR_INVALID;
  if (n > 0 && (!x_bf16 || !aligned16(x_bf16))) return FP8_ERR_INVALID;
  return hip_status(launch_amax(x_bf16, n, s_dev, true, fmt, margin, mu_log2, stream));
}

int32_t fp8_bias_host(float amax, fp8_fmt fmt, int margin, int mu_log2, uint32_t* flags_out) {
  uint32_t bits;
  memcpy(&bits, &amax, 4);
  if (margin > kIntArgLimit) margin = kIntArgLimit;
  if (margin < -kIntArgLimit) margin = -kIntArgLimit;
  if (mu_log2 > kIntArgLimit) mu_log2 = kIntArgLimit;
  if (mu_log2 < -kIntArgLimit) mu_log2 = -kIntArgLimit;
  return bias_from_amax_bits(bits & 0x7FFFFFFFu, fmt, margin, mu_log2, flags_out);
}

fp8_status fp8_scale_fixed(fp8_scale_t* s_dev, int32_t bias, hipStream_t stream) {
  if (!s_dev || !aligned16(s_dev) || bias < -126 || bias > 126) return FP8_ERR_INVALID;
  return hip_status(launch_scale_fixed(s_dev, bias, stream));
}

fp8_status fp8_cast(const void* x_bf16, int64_t rows, int64_t cols, fp8_fmt fmt,
                    const fp8_scale_t* s_dev, uint8_t* out_rowwise, uint8_t* out_transposed,
                    hipStream_t stream) {
  if (rows < 0 || cols < 0 || !fmt_ok(fmt) || !s_dev || !aligned16(s_dev)) return FP8_ERR_INVALID;
  if (rows % 16 || cols % 16 || rows >= kMaxDim || cols >= kMaxDim) return FP8_ERR_UNSUPPORTED;
  if (rows > 0 && cols > 0) {
    if (!x_bf16 || !aligned16(x_bf16)) return FP8_ERR_INVALID;
    if (out_rowwise && !aligned16(out_rowwise)) return FP8_ERR_INVALID;
    if (out_transposed && !aligned16(out_transposed)) return FP8_ERR_INVALID;
  }
  return hip_status(launch_cast(x_bf16, rows, cols, fmt, s_dev, out_rowwise, out_transposed, stream));
}

// the argument checks of fp8_quantize
static fp8_status check_quantize(const void* x_bf16, int64_t rows, int64_t cols, int fmt, int margin, int mu_log2,
                                 const fp8_scale_t* s_dev, const uint8_t* out_rowwise,
                                 const uint8_t* out_transposed) {
  if (rows < 0 || cols < 0 || !fmt_ok(fmt) || !int_ok(margin) || !int_ok(mu_log2) || !s_dev ||
      !aligned16(s_dev))
    return FP8_ERR_INVALID;
  if (rows % 16 || cols % 16 || rows >= kMaxDim || cols >= kMaxDim) return FP8_ERR_UNSUPPORTED;
  if (rows > 0 && cols > 0) {
    if (!x_bf16 || !aligned16(x_bf16)) return FP8_ERR_INVALID;
    if (out_rowwise && !aligned16(out_rowwise)) return FP8_ERR_INVALID;
    if (out_transposed && !aligned16(out_transposed)) return FP8_ERR_INVALID;
  }
  return FP8_OK;
}

fp8_status fp8_quantize(const void* x_bf16, int64_t rows, int64_t cols, fp8_fmt fmt, int margin,
                        int mu_log2, fp8_scale_t* s_dev, uint8_t* out_rowwise, uint8_t* out_transposed,
                        hipStream_t stream) {
  const fp8_status st = check_quantize(x_bf16, rows, cols, fmt, margin, mu_log2, s_dev, out_rowwise, out_transposed);
  if (st != FP8_OK) return st;
  return hip_status(launch_quantize(x_bf16, rows, cols, fmt, margin, mu_log2, s_dev, out_rowwise,
                                    out_transposed, stream));
}

fp8_status fp8_quantize_spec(const void* x_bf16, int64_t rows, int64_t cols, fp8_fmt fmt, int margin,
                             int mu_log2, fp8_scale_t* s_dev, uint8_t* out_rowwise, hipStream_t stream) {
  const fp8_status st = check_quantize(x_bf16, rows, cols, fmt, margin, mu_log2, s_dev, out_rowwise, nullptr);
  if (st != FP8_OK) return st;
  if (rows > 0 && cols > 0 && !out_rowwise) return FP8_ERR_INVALID;
  return hip_status(launch_quantize_spec(x_bf16, rows, cols, fmt, margin, mu_log2, s_dev, out_rowwise, stream));
}

fp8_status fp8_quantize_batch(const fp8_quantize_args* tensors, int count, hipStream_t stream) {
  if (!tensors || count < 1 || count > FP8_QUANTIZE_BATCH_MAX) return FP8_ERR_INVALID;
  static_assert(FP8_QUANTIZE_BATCH_MAX == kQuantBatchMax, "batch limit");
  QuantDesc d[kQuantBatchMax];
  for (int i = 0; i < count; ++i) {
    const fp8_quantize_args& a = tensors[i];
    const fp8_status st = check_quantize(a.x, a.rows, a.cols, a.fmt, a.margin, a.mu_log2, a.s, a.out_rowwise,
                                         a.out_transposed);
    if (st != FP8_OK) return st;
    for (int k = 0; k < i; ++k)
      if (tensors[k].s == a.s) return FP8_ERR_INVALID;  // one record per tensor
    d[i] = QuantDesc{a.x, a.rows, a.cols, (int)a.fmt, a.margin, a.mu_log2, a.s, a.out_rowwise, a.out_transposed};
  }
  return hip_status(launch_quantize_batch(d, count, stream));
}

// the argument checks of fp8_gemm
static fp8_status check_gemm(const uint8_t* A, int fa, int la, const fp8_scale_t* sa, const uint8_t* B, int fb,
                             int lb, const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R, const void* C_bf16) {
  if (M < 0 || N < 0 || R < 0 || !fmt_ok(fa) || !fmt_ok(fb)) return FP8_ERR_INVALID;
  if ((la != FP8_OPERAND_ROWS && la != FP8_OPERAND_COLS) || (lb != FP8_OPERAND_ROWS && lb != FP8_OPERAND_COLS))
    return FP8_ERR_INVALID;
  if (!sa || !sb || !aligned16(sa) || !aligned16(sb)) return FP8_ERR_INVALID;
  if (M % 16 || N % 16 || R % 16 || M >= kMaxDim || N >= kMaxDim || R >= kMaxDim || !gemm_fits(M, N, R))
    return FP8_ERR_UNSUPPORTED;
  if (M > 0 && N > 0) {
    if (!C_bf16 || !aligned16(C_bf16)) return FP8_ERR_INVALID;
    if (R > 0 && (!A || !B || !aligned16(A) || !aligned16(B))) return FP8_ERR_INVALID;
  }
  return FP8_OK;
}

fp8_status fp8_gemm(const uint8_t* A, fp8_fmt fa, fp8_layout la, const fp8_scale_t* sa, const uint8_t* B,
                    fp8_fmt fb, fp8_layout lb, const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R,
                    void* C_bf16, hipStream_t stream) {
  const fp8_status st = check_gemm(A, fa, la, sa, B, fb, lb, sb, M, N, R, C_bf16);
  if (st != FP8_OK) return st;
  return hip_status(launch_gemm(A, fa, la == FP8_OPERAND_COLS, sa, B, fb, lb == FP8_OPERAND_COLS, sb, M, N, R,
                                C_bf16, stream));
}

size_t fp8_gemm_workspace_bytes(fp8_fmt fa, fp8_fmt fb, int64_t M, int64_t N, int64_t R, fp8_split split) {
  if (M < 0 || N < 0 || R < 0) return 0;
  return gemm_tail_split((int)fa, (int)fb, M, N, R, (int)split).bytes;
}

fp8_status fp8_gemm_ws(const uint8_t* A, fp8_fmt fa, fp8_layout la, const fp8_scale_t* sa, const uint8_t* B,
                       fp8_fmt fb, fp8_layout lb, const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R,
                       void* C_bf16, fp8_split split, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const fp8_status st = check_gemm(A, fa, la, sa, B, fb, lb, sb, M, N, R, C_bf16);
  if (st != FP8_OK) return st;
  if (split != FP8_SPLIT_AUTO && split != FP8_SPLIT_NEVER && split != FP8_SPLIT_TAIL) return FP8_ERR_INVALID;
  if (workspace && !aligned16(workspace)) return FP8_ERR_INVALID;
  return hip_status(launch_gemm_ws(A, fa, la == FP8_OPERAND_COLS, sa, B, fb, lb == FP8_OPERAND_COLS, sb, M, N, R,
                                   C_bf16, (int)split, workspace, workspace_bytes, stream));
}

fp8_status fp8_gemm_noalloc(const uint8_t* A, fp8_fmt fa, fp8_layout la, const fp8_scale_t* sa, const uint8_t* B,
                            fp8_fmt fb, fp8_layout lb, const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R,
                            void* C_bf16, fp8_split split, hipStream_t stream) {
  const fp8_status st = check_gemm(A, fa, la, sa, B, fb, lb, sb, M, N, R, C_bf16);
  if (st != FP8_OK) return st;
  if (split != FP8_SPLIT_AUTO && split != FP8_SPLIT_NEVER && split != FP8_SPLIT_TAIL) return FP8_ERR_INVALID;
  void* ws = nullptr;
  size_t cap = 0;
  if (static_scratch(&ws, &cap) != hipSuccess) return FP8_ERR_HIP;
  if (gemm_tail_split(fa, fb, M, N, R, (int)split).bytes > cap) return FP8_ERR_UNSUPPORTED;
  return hip_status(launch_gemm_ws(A, fa, la == FP8_OPERAND_COLS, sa, B, fb, lb == FP8_OPERAND_COLS, sb, M, N, R,
                                   C_bf16, (int)split, ws, cap, stream));
}

fp8_status fp8_gemm_pair(const fp8_gemm_args* first, const fp8_gemm_args* second, hipStream_t stream) {
  if (!first || !second) return FP8_ERR_INVALID;
  GemmDesc g[2];
  const fp8_gemm_args* a[2] = {first, second};
  for (int i = 0; i < 2; ++i) {
    const fp8_gemm_args& x = *a[i];
    const fp8_status st = check_gemm(x.A, x.fa, x.la, x.sa, x.B, x.fb, x.lb, x.sb, x.M, x.N, x.R, x.C);
    if (st != FP8_OK) return st;
    g[i] = GemmDesc{x.A, (int)x.fa, x.la == FP8_OPERAND_COLS, x.sa, x.B, (int)x.fb, x.lb == FP8_OPERAND_COLS,
                    x.sb, x.M, x.N, x.R, x.C};
  }
  return hip_status(launch_gemm_pair(g[0], g[1], stream));
}

fp8_status fp8_gemm_nt(const uint8_t* A, fp8_fmt fa, const fp8_scale_t* sa, const uint8_t* B,
                       fp8_fmt fb, const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R,
                       void* C_bf16, hipStream_t stream) {
  return fp8_gemm(A, fa, FP8_OPERAND_ROWS, sa, B, fb, FP8_OPERAND_ROWS, sb, M, N, R, C_bf16, stream);
}

// required: x8, w8, sx, sw (and dy8, sdy for the backward); optional
// (NULL or aligned): the transposed copies x8t, w8t, dy8t
static fp8_status check_ws(const fp8_linear_ws* ws, bool fwd) {
  if (!ws) return FP8_ERR_INVALID;
  const void* p[] = {ws->x8, ws->w8, ws->sx, ws->sw, fwd ? (const void*)ws->x8 : (const void*)ws->dy8,
                     fwd ? (const void*)ws->x8 : (const void*)ws->sdy};
  for (const void* q : p)
    if (!q || !aligned16(q)) return FP8_ERR_INVALID;
  const void* o[] = {ws->x8t, ws->w8t, ws->dy8t, ws->scratch};
  for (const void* q : o)
    if (q && !aligned16(q)) return FP8_ERR_INVALID;
  return FP8_OK;
}

fp8_status fp8_linear_fwd(const void* X, const void* W, int64_t M, int64_t K, int64_t N, int margin,
                          const fp8_linear_ws* ws, void* Y, hipStream_t stream) {
  if (M < 0 || K < 0 || N < 0 || !int_ok(margin)) return FP8_ERR_INVALID;
  if (M % 16 || K % 16 || N % 16 || M >= kMaxDim || K >= kMaxDim || N >= kMaxDim ||
      !gemm_fits(M, N, K) || !gemm_fits(K, N, M))
    return FP8_ERR_UNSUPPORTED;
  fp8_status st = check_ws(ws, true);
  if (st != FP8_OK) return st;
  if ((M * K > 0 && (!X || !aligned16(X))) || (K * N > 0 && (!W || !aligned16(W))) ||
      (M * N > 0 && (!Y || !aligned16(Y))))
    return FP8_ERR_INVALID;
  if (ws->sx == ws->sw) return FP8_ERR_INVALID;
  // X and W in one amax launch and one cast launch
  const QuantDesc q[2] = {QuantDesc{X, M, K, FP8_E4M3, margin, 0, ws->sx, ws->x8, ws->x8t},
                          QuantDesc{W, K, N, FP8_E4M3, margin, 0, ws->sw, ws->w8, ws->w8t}};
  if (launch_quantize_batch(q, 2, stream) != hipSuccess) return FP8_ERR_HIP;
  // Y[m, n] = sum_k x8[m, k] w8[k, n]: w8 read reduction-major (last wave
  // split over the scratch workspace when it is given and large enough)
  return hip_status(launch_gemm_ws(ws->x8, FP8_E4M3, false, ws->sx, ws->w8, FP8_E4M3, true, ws->sw, M, N, K, Y,
                                   FP8_SPLIT_AUTO, ws->scratch, ws->scratch_bytes, stream));
}

size_t fp8_linear_scratch_bytes(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K < 0 || N < 0) return 0;
  return gemm_tail_split(FP8_E4M3, FP8_E4M3, M, N, K, FP8_SPLIT_AUTO).bytes;
}

fp8_status fp8_linear_bwd(const void* dY, int64_t M, int64_t K, int64_t N, int margin, int mu_log2,
                          const fp8_linear_ws* ws, void* dX, void* dW, hipStream_t stream) {
  if (M < 0 || K < 0 || N < 0 || !int_ok(margin) || !int_ok(mu_log2)) return FP8_ERR_INVALID;
  if (M % 16 || K % 16 || N % 16 || M >= kMaxDim || K >= kMaxDim || N >= kMaxDim ||
      !gemm_fits(M, K, N) || !gemm_fits(K, N, M))
    return FP8_ERR_UNSUPPORTED;
  fp8_status st = check_ws(ws, false);
  if (st != FP8_OK) return st;
  if ((M * N > 0 && (!dY || !aligned16(dY))) || (dX && !aligned16(dX)) || (dW && !aligned16(dW)))
    return FP8_ERR_INVALID;
  // dY's quantise rewrites sdy, which the GEMMs read beside sx and sw
  if (ws->sdy == ws->sx || ws->sdy == ws->sw) return FP8_ERR_INVALID;
  hipError_t e;
  if ((e = launch_quantize(dY, M, N, FP8_E5M2, margin, mu_log2, ws->sdy, ws->dy8, ws->dy8t,
                           stream)) != hipSuccess)
    return FP8_ERR_HIP;
  // dX[m, k] = sum_n dy8[m, n] w8[k, n]; dW[k, n] = sum_m x8[m, k] dy8[m, n]
  // (both read reduction-major); when both are asked for, one launch
  const GemmDesc dgrad{ws->dy8, FP8_E5M2, false, ws->sdy, ws->w8, FP8_E4M3, false, ws->sw, M, K, N, dX};
  const GemmDesc wgrad{ws->x8, FP8_E4M3, true, ws->sx, ws->dy8, FP8_E5M2, true, ws->sdy, K, N, M, dW};
  if (dX && dW) e = launch_gemm_pair(dgrad, wgrad, stream);
  else if (dX) e = launch_gemm(dgrad.A, dgrad.fa, dgrad.ta, dgrad.sa, dgrad.B, dgrad.fb, dgrad.tb, dgrad.sb, M, K, N,
                               dX, stream);
  else if (dW) e = launch_gemm(wgrad.A, wgrad.fa, wgrad.ta, wgrad.sa, wgrad.B, wgrad.fb, wgrad.tb, wgrad.sb, K, N, M,
                               dW, stream);
  return hip_status(e);
}

fp8_status fp8_linear_fwd_cached(const void* X, int64_t M, int64_t K, int64_t N, int margin,
                                 fp8_scaling x_scaling, const uint8_t* w8, fp8_layout lw, const fp8_scale_t* sw,
                                 uint8_t* x8, fp8_scale_t* sx, void* Y, hipStream_t stream) {
  if (M < 0 || K < 0 || N < 0 || !int_ok(margin)) return FP8_ERR_INVALID;
  if (x_scaling != FP8_SCALING_AMAX && x_scaling != FP8_SCALING_FIXED) return FP8_ERR_INVALID;
  if (lw != FP8_OPERAND_ROWS && lw != FP8_OPERAND_COLS) return FP8_ERR_INVALID;
  if (!sw || !aligned16(sw) || !sx || !aligned16(sx)) return FP8_ERR_INVALID;
  if (sx == sw) return FP8_ERR_INVALID;  // X's quantise would rewrite the weight's record
  if (M % 16 || K % 16 || N % 16 || M >= kMaxDim || K >= kMaxDim || N >= kMaxDim || !gemm_fits(M, N, K))
    return FP8_ERR_UNSUPPORTED;
  if ((M * K > 0 && (!X || !aligned16(X) || !x8 || !aligned16(x8))) ||
      (N * K > 0 && (!w8 || !aligned16(w8))) || (M * N > 0 && (!Y || !aligned16(Y))))
    return FP8_ERR_INVALID;
  hipError_t e = x_scaling == FP8_SCALING_AMAX
                     ? launch_quantize(X, M, K, FP8_E4M3, margin, 0, sx, x8, nullptr, stream)
                     : launch_cast(X, M, K, FP8_E4M3, sx, x8, nullptr, stream);
  if (e != hipSuccess) return FP8_ERR_HIP;
  return hip_status(launch_gemm(x8, FP8_E4M3, false, sx, w8, FP8_E4M3, lw == FP8_OPERAND_COLS, sw, M, N, K, Y,
                                stream));
}

fp8_status fp8_wgrad_fp8(const uint8_t* x8, fp8_layout lx, const fp8_scale_t* sx, const uint8_t* dy8,
                         fp8_layout ldy, const fp8_scale_t* sdy, int64_t K, int64_t N, int64_t M, int margin,
                         int mu_log2, void* dW_bf16, fp8_scale_t* s_dw, uint8_t* dw8, uint8_t* dw8t,
                         hipStream_t stream) {
  if (K < 0 || N < 0 || M < 0 || !int_ok(margin) || !int_ok(mu_log2)) return FP8_ERR_INVALID;
  if ((lx != FP8_OPERAND_ROWS && lx != FP8_OPERAND_COLS) || (ldy != FP8_OPERAND_ROWS && ldy != FP8_OPERAND_COLS))
    return FP8_ERR_INVALID;
  if (!sx || !aligned16(sx) || !sdy || !aligned16(sdy) || !s_dw || !aligned16(s_dw)) return FP8_ERR_INVALID;
  if (K % 16 || N % 16 || M % 16 || K >= kMaxDim || N >= kMaxDim || M >= kMaxDim || !gemm_fits(K, N, M))
    return FP8_ERR_UNSUPPORTED;
  if (K > 0 && N > 0) {
    if (!dW_bf16 || !aligned16(dW_bf16) || !dw8 || !aligned16(dw8)) return FP8_ERR_INVALID;
    if (dw8t && !aligned16(dw8t)) return FP8_ERR_INVALID;
    if (M > 0 && (!x8 || !aligned16(x8) || !dy8 || !aligned16(dy8))) return FP8_ERR_INVALID;
  }
  hipError_t e = K > 0 && N > 0
                     ? launch_gemm_wgrad_amax(x8, lx == FP8_OPERAND_COLS, sx, dy8, ldy == FP8_OPERAND_COLS, sdy, K,
                                              N, M, dW_bf16, s_dw, stream)
                     : launch_amax_gen(nullptr, 0, s_dw, stream);  // an empty max, so the record publishes
  if (e != hipSuccess) return FP8_ERR_HIP;
  return hip_status(launch_wgrad_cast(dW_bf16, K, N, s_dw, dw8, dw8t, margin, mu_log2, stream));
}

fp8_status fp8_adam_init_master(int64_t n, const void* w_bf16, uint16_t* w16, fp8_scale_t* s_w, hipStream_t stream) {
  if (n < 0 || !s_w || !aligned16(s_w)) return FP8_ERR_INVALID;
  if (n % 16) return FP8_ERR_UNSUPPORTED;
  if (n > 0 && (!w_bf16 || !aligned16(w_bf16) || !w16 || !aligned16(w16))) return FP8_ERR_INVALID;
  return hip_status(launch_master_init(n, (const uint16_t*)w_bf16, w16, s_w, stream));
}

fp8_status fp8_adam_step(int64_t n, const uint8_t* g8, const fp8_scale_t* s_g, uint8_t* m1, fp8_scale_t* s_m1,
                         uint16_t* m2, fp8_scale_t* s_m2, uint16_t* w16, fp8_scale_t* s_w, void* w_bf16, float lr,
                         float beta1, float beta2, float eps, float weight_decay, int32_t step, hipStream_t stream) {
  AdamHyper h;
  const fp8_status st = adam_check(n, g8, s_g, m1, s_m1, m2, s_m2, w16, s_w, w_bf16, lr, beta1, beta2, eps,
                                   weight_decay, step, h);
  if (st != FP8_OK) return st;
  return hip_status(launch_adam(n, g8, s_g, m1, s_m1, m2, s_m2, w16, s_w, (uint16_t*)w_bf16, h, stream));
}

fp8_status fp8_adam_step_spec(int64_t n, const uint8_t* g8, const fp8_scale_t* s_g, const uint8_t* m1,
                              const uint16_t* m2, const uint16_t* w16, uint8_t* m1_out, uint16_t* m2_out,
                              uint16_t* w16_out, fp8_scale_t* s_m1, fp8_scale_t* s_m2, fp8_scale_t* s_w,
                              void* w_bf16, uint32_t* missed, float lr, float beta1, float beta2, float eps,
                              float weight_decay, int32_t step, hipStream_t stream) {
  AdamHyper h;
  const fp8_status st = adam_check(n, g8, s_g, m1, s_m1, m2, s_m2, w16, s_w, w_bf16, lr, beta1, beta2, eps,
                                   weight_decay, step, h);
  if (st != FP8_OK) return st;
  if (missed && !aligned4(missed)) return FP8_ERR_INVALID;
  if (n > 0) {
    // outputs: present, aligned, and disjoint from every input and from each other
    const Range outs[] = {{m1_out, (size_t)n}, {m2_out, 2 * (size_t)n}, {w16_out, 2 * (size_t)n},
                          {w_bf16, w_bf16 ? 2 * (size_t)n : 0}};
    const Range ins[] = {{g8, (size_t)n}, {m1, (size_t)n}, {m2, 2 * (size_t)n}, {w16, 2 * (size_t)n}};
    for (int i = 0; i < 3; ++i)
      if (!outs[i].p || !aligned16(outs[i].p)) return FP8_ERR_INVALID;
    for (const Range& o : outs) {
      for (const Range& q : ins)
        if (overlaps(o, q)) return FP8_ERR_INVALID;
      for (const Range& q : outs)
        if (&q != &o && overlaps(o, q)) return FP8_ERR_INVALID;
    }
  }
  return hip_status(launch_adam_spec(n, g8, s_g, m1, m2, w16, m1_out, m2_out, w16_out, s_m1, s_m2, s_w,
                                     (uint16_t*)w_bf16, missed, h, stream));
}

}  // extern "C"
