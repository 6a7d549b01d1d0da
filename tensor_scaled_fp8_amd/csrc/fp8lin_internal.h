// Internal declarations shared by the HIP sources of libfp8lin.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8lin.h"

namespace fp8lin {

// Largest finite value of each format is 1.75 * 2^kTopExp.
constexpr int kTopExpE4M3 = 8;   // 448
constexpr int kTopExpE5M2 = 15;  // 57344
constexpr int kBiasMin = -126;
constexpr int kBiasMax = 126;
constexpr int kIntArgLimit = 1024;

// Scale choice from amax, given as the bit pattern of |amax| in fp32
// (0..0x7FFFFFFF; a bf16 amax is its 16-bit pattern shifted left by 16):
//   bias = floor(log2(fmt_max / amax)) - margin + mu_log2, clamped.
// Writing amax = m * 2^e with m in [1, 2) and fmt_max = 1.75 * 2^E, the
// floor is E - e when m <= 1.75 and E - e - 1 when m > 1.75, so the rule
// needs only the exponent and mantissa fields: no floating-point log.
__host__ __device__ inline int32_t bias_from_amax_bits(uint32_t mag, int fmt, int margin, int mu_log2,
                                                       uint32_t* flags) {
  uint32_t f = 0;
  int32_t b = 0;
  if (mag >= 0x7F800000u) {
    f = FP8_FLAG_NONFINITE;
  } else if (mag == 0u) {
    f = FP8_FLAG_ZERO;
  } else {
    const int top = (fmt == FP8_E5M2) ? kTopExpE5M2 : kTopExpE4M3;
    const uint32_t ef = mag >> 23, mf = mag & 0x7FFFFFu;
    int e;
    bool above;  // significand > 1.75
    if (ef != 0) {
      e = (int)ef - 127;
      above = mf > 0x600000u;  // 1 + mf/2^23 > 1.75
    } else {
      // subnormal: mf * 2^-149 = 2^(p-149) * (mf / 2^p), p = highest set bit
      const int p = 31 - __builtin_clz(mf);
      e = p - 149;
      above = 4u * mf > (7u << p);  // mf / 2^p > 1.75
    }
    b = top - e - (above ? 1 : 0) - margin + mu_log2;
    if (b < kBiasMin || b > kBiasMax) {
      f |= FP8_FLAG_CLAMPED;
      b = b < kBiasMin ? kBiasMin : kBiasMax;
    }
  }
  if (flags) *flags = f;
  return b;
}

// The same rule for an FP16 store (max 65504 = (2 - 2^-10) * 2^15), margin 0:
// the floor is 15 - e when the significand is <= 2 - 2^-10, else 14 - e.
__host__ __device__ inline int32_t bias_fp16_from_amax_bits(uint32_t mag, uint32_t* flags) {
  uint32_t f = 0;
  int32_t b = 0;
  if (mag >= 0x7F800000u) {
    f = FP8_FLAG_NONFINITE;
  } else if (mag == 0u) {
    f = FP8_FLAG_ZERO;
  } else {
    const uint32_t ef = mag >> 23, mf = mag & 0x7FFFFFu;
    int e;
    bool above;  // significand > 2 - 2^-10
    if (ef != 0) {
      e = (int)ef - 127;
      above = mf > 0x7FE000u;
    } else {
      const int p = 31 - __builtin_clz(mf);
      e = p - 149;
      above = 1024ull * mf > (2047ull << p);
    }
    b = 15 - e - (above ? 1 : 0);
    if (b < kBiasMin || b > kBiasMax) {
      f |= FP8_FLAG_CLAMPED;
      b = b < kBiasMin ? kBiasMin : kBiasMax;
    }
  }
  if (flags) *flags = f;
  return b;
}

// Tag under which a reduction merges this call's maximum into s->gen_max:
// one above the record's epoch. Only the kernel that consumes the maximum
// advances epoch (to gen_max >> 16), after the reduction kernel has
// finished, so every block of a reduction reads the same value.
__device__ inline unsigned long long reduction_tag(const fp8_scale_t* s) {
  return __hip_atomic_load((const unsigned long long*)&s->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) +
         1ull;
}

__host__ __device__ inline float pow2f(int32_t b) {  // 2^b for b in [-126, 127]
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)(b + 127) << 23;
  return v.f;
}

// Kernel launchers (defined in the .hip files). They assume validated
// arguments and return the launch status.
hipError_t launch_scale_reset(fp8_scale_t* s, int64_t count, hipStream_t st);
hipError_t launch_amax(const void* x, int64_t n, fp8_scale_t* s, bool fuse_scale, int fmt, int margin,
                       int mu_log2, hipStream_t st);
hipError_t launch_scale(fp8_scale_t* s, int fmt, int margin, int mu_log2, hipStream_t st);
hipError_t launch_scale_fixed(fp8_scale_t* s, int32_t bias, hipStream_t st);
hipError_t launch_cast(const void* x, int64_t rows, int64_t cols, int fmt, const fp8_scale_t* s,
                       uint8_t* out_row, uint8_t* out_t, hipStream_t st);
// tagged amax reduction into s->gen_max (see reduction_tag)
hipError_t launch_amax_gen(const void* x, int64_t n, fp8_scale_t* s, hipStream_t st);
// amax pass + cast that derives the scale (fp8_quantize)
hipError_t launch_quantize(const void* x, int64_t rows, int64_t cols, int fmt, int margin, int mu_log2,
                           fp8_scale_t* s, uint8_t* out_row, uint8_t* out_t, hipStream_t st);
// fp8_quantize_spec: one pass that casts with the record's current bias and
// merges the amax, then a check that recasts only if the bias changed
// (row-major output only)
hipError_t launch_quantize_spec(const void* x, int64_t rows, int64_t cols, int fmt, int margin, int mu_log2,
                                fp8_scale_t* s, uint8_t* out_row, hipStream_t st);
// Several tensors quantised in two launches (fp8_quantize_batch).
constexpr int kQuantBatchMax = 4;
struct QuantDesc {
  const void* x;
  int64_t rows, cols;
  int fmt, margin, mu_log2;
  fp8_scale_t* s;
  uint8_t* out_row;
  uint8_t* out_t;
};
// the amax passes of count tensors (1..kQuantBatchMax, distinct records) in one launch
hipError_t launch_amax_batch(const QuantDesc* d, int count, hipStream_t st);
// amax passes, then the derive-casts, each tensor as launch_quantize would do it
hipError_t launch_quantize_batch(const QuantDesc* d, int count, hipStream_t st);
// ta / tb: operand stored reduction-major (A [R, M], B [R, N]) instead of
// one row per output index (A [M, R], B [N, R])
hipError_t launch_gemm(const uint8_t* A, int fa, bool ta, const fp8_scale_t* sa, const uint8_t* B, int fb, bool tb,
                       const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R, void* C,
                       hipStream_t st);
// Tail split of a forward-format GEMM (E4M3 x E4M3, R a multiple of 256):
// when the tiles leave a last wave at most half full, those ntail tiles
// are computed in two reduction halves each (FP32 partials in a caller
// workspace of `bytes`) and summed by a fixup kernel, after the nfull
// tiles of the whole waves. mode: FP8_SPLIT_AUTO also needs R >= 16384
// (the fixup launch and the partials' traffic cost more than half a
// shorter tile), FP8_SPLIT_TAIL only R >= 512, FP8_SPLIT_NEVER never.
// ntail = 0: no split for this shape on the current device.
struct TailSplit {
  int nfull, ntail;
  size_t bytes;
};
constexpr int64_t kSplitMinR = 16384;
TailSplit gemm_tail_split(int fa, int fb, int64_t M, int64_t N, int64_t R, int mode);
// launch_gemm, with the tail split when gemm_tail_split plans one and the
// workspace holds its partials (else exactly launch_gemm)
hipError_t launch_gemm_ws(const uint8_t* A, int fa, bool ta, const fp8_scale_t* sa, const uint8_t* B, int fb,
                          bool tb, const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R, void* C, int mode,
                          void* ws, size_t ws_bytes, hipStream_t st);
// The device's static scratch of fp8_gemm_noalloc (its address on the
// current device, looked up once per device, and its size in bytes): room
// for the tail split of kStaticTailTiles tiles, the most a last wave at
// most half full holds on a 256-CU device.
constexpr int kStaticTailTiles = 128;
constexpr int kMaxDevices = 64;
hipError_t static_scratch(void** ptr, size_t* bytes);
// One GEMM of a pair (the arguments of launch_gemm).
struct GemmDesc {
  const uint8_t* A;
  int fa;
  bool ta;
  const fp8_scale_t* sa;
  const uint8_t* B;
  int fb;
  bool tb;
  const fp8_scale_t* sb;
  int64_t M, N, R;
  void* C;
};
// true when the pair has a one-launch kernel: the linear backward's dgrad
// (E5M2 x E4M3, both one row per output index) then its wgrad (E4M3 x
// E5M2, both reduction-major)
bool gemm_pair_fused(const GemmDesc& g0, const GemmDesc& g1);
// both GEMMs, bit-identical to two launch_gemm calls: one launch when
// gemm_pair_fused, else two
hipError_t launch_gemm_pair(const GemmDesc& g0, const GemmDesc& g1, hipStream_t st);
hipError_t launch_gemm_wgrad_amax(const uint8_t* A, bool ta, const fp8_scale_t* sa, const uint8_t* B, bool tb,
                                  const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R, void* C,
                                  fp8_scale_t* s_out, hipStream_t st);
// E5M2 derive-cast of a weight gradient whose amax the wgrad GEMM merged,
// counting saturated elements into s->sat_count
hipError_t launch_wgrad_cast(const void* dw, int64_t rows, int64_t cols, fp8_scale_t* s, uint8_t* out_row,
                             uint8_t* out_t, int margin, int mu_log2, hipStream_t st);

struct AdamHyper {
  float lr, beta1, beta2, eps, weight_decay, bc1, bc2;  // bc = 1 / (1 - beta^step)
};
hipError_t launch_adam(int64_t n, const uint8_t* g8, const fp8_scale_t* s_g, uint8_t* m1, fp8_scale_t* s_m1,
                       uint16_t* m2, fp8_scale_t* s_m2, uint16_t* w, fp8_scale_t* s_w, uint16_t* w_bf16,
                       const AdamHyper& h, hipStream_t st);
hipError_t launch_adam_spec(int64_t n, const uint8_t* g8, const fp8_scale_t* s_g, const uint8_t* m1,
                            const uint16_t* m2, const uint16_t* w, uint8_t* m1_out, uint16_t* m2_out, uint16_t* w_out,
                            fp8_scale_t* s_m1, fp8_scale_t* s_m2, fp8_scale_t* s_w, uint16_t* w_bf16,
                            uint32_t* missed, const AdamHyper& h, hipStream_t st);
hipError_t launch_master_init(int64_t n, const uint16_t* w_bf16, uint16_t* w, fp8_scale_t* s_w, hipStream_t st);

}  // namespace fp8lin
