// O2 precision-decoupled Adam step (AdamW form) on scaled low-precision
// optimizer state.
//
// [FP8-LM reading note, "Proposed method", O2] the optimizer's auxiliary
// tensors go to low precision with precision decoupling: the first moment
// in FP8, the second moment in FP16, the master weights in FP16 with tensor
// scaling (6 bytes per parameter with the FP8 gradient); the ablation keeps
// master weights and the second moment at FP16 or above. Readings where the
// page is silent: the FP8 first moment is E4M3; the second moment carries a
// per-tensor power-of-two scale as the master weights do (squared gradients
// of the size the FP8 gradient path emits, ~1e-10, lie below FP16's
// subnormal range); each new per-tensor scale is chosen just in time from
// the new tensor's max |value| with the rule of the FP8 path (largest power
// of two that keeps it within the format's max); AdamW with bias correction.
//
// Three launches, all on the caller's stream:
//  1. pass 1: the update of every element in fp32, max |m1'|, max m2',
//     max |w'| merged into each record's reduce_bits (fp32 magnitude bits,
//     one device-scope atomic max per block).
//  2. pass 2: the same update recomputed (one shared function, contraction
//     off, explicit FMAs, so the values equal pass 1's), encoded with the new
//     scales derived from reduce_bits and written in place; the old scales
//     are still the records' public fields, which nothing changes before
//     this pass ends.
//  3. publish (one thread): the new public fields of the three records;
//     reduce_bits back to 0 for the next step.
// HBM traffic per parameter: 6 bytes read twice, 5 written (+2 for the bf16
// copy of the weights for the next forward).
//
// One-pass variant (launch_adam_spec), out of place: a new scale is almost
// always the one the record already holds (a tensor's max moves across a
// power of two only now and then), so the first kernel encodes with the
// records' current scales while it takes the maxima, writing the new state
// to separate buffers (6 bytes read, 5 + 2 written). The second kernel
// derives the new scales; where all three equal the current ones it
// returns at once, else it recomputes every element from the untouched
// inputs with the new scales. Either way the stored state is bit for bit
// what the two-pass step stores, since both encode the same fp32 values
// with the same scale.
#include "fp8lin_internal.h"

namespace fp8lin {
namespace {

constexpr int kThreads = 1024;        // 16 waves per block: many resident waves, few blocks
constexpr int kVec = 8;           // elements per thread per iteration
constexpr int kMaxBlocks = 512;      // one max merge per block and record

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct Vals {
  float m1, m2, w;
};

// One element of the update, in fp32. Same instructions in both passes.
// The square root and the reciprocal are the hardware approximations
// (v_sqrt_f32, v_rcp_f32, about 1 ulp each): correctly rounded division and
// square root made the pass ALU-bound, and the update needs no more than
// fp32 accuracy.
__device__ inline Vals adam_update(float g, float m1, float m2, float w, const AdamHyper& h) {
#pragma clang fp contract(off)
  const float m1n = __builtin_fmaf(h.beta1, m1, (1.0f - h.beta1) * g);
  const float m2n = __builtin_fmaf(h.beta2, m2, ((1.0f - h.beta2) * g) * g);
  const float mh = m1n * h.bc1;
  const float vh = m2n * h.bc2;
  const float step = mh * __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(vh) + h.eps) + h.weight_decay * w;
  Vals r;
  r.m1 = m1n;
  r.m2 = m2n;
  r.w = w - h.lr * step;
  return r;
}

// the four FP8 values of a word (byte order = element order)
__device__ inline void dec_e5m2x4(uint32_t w, float f[4]) {
  f[0] = __builtin_amdgcn_cvt_f32_bf8((int)w, 0);
  f[1] = __builtin_amdgcn_cvt_f32_bf8((int)w, 1);
  f[2] = __builtin_amdgcn_cvt_f32_bf8((int)w, 2);
  f[3] = __builtin_amdgcn_cvt_f32_bf8((int)w, 3);
}
__device__ inline void dec_e4m3x4(uint32_t w, float f[4]) {
  f[0] = __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
  f[1] = __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
  f[2] = __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
  f[3] = __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
}
__device__ inline float dec_f16(uint32_t word, int half) {
  const uint16_t h = (uint16_t)(half ? word >> 16 : word & 0xFFFFu);
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ inline uint32_t enc_f16x2(float a, float b) {
  const uint16_t ha = __builtin_bit_cast(uint16_t, (_Float16)a);
  const uint16_t hb = __builtin_bit_cast(uint16_t, (_Float16)b);
  return (uint32_t)ha | ((uint32_t)hb << 16);
}

// the 8 updated elements of one thread's chunk
__device__ inline void update8(u32x2 gw, u32x2 m1w, u32x4 m2w, u32x4 ww, float g_inv, float m1_inv, float m2_inv,
                               float w_inv, const AdamHyper& h, Vals out[kVec]) {
  float g[8], m1[8];
  dec_e5m2x4(gw.x, &g[0]);
  dec_e5m2x4(gw.y, &g[4]);
  dec_e4m3x4(m1w.x, &m1[0]);
  dec_e4m3x4(m1w.y, &m1[4]);
  const uint32_t m232[4] = {m2w.x, m2w.y, m2w.z, m2w.w}, w32[4] = {ww.x, ww.y, ww.z, ww.w};
#pragma unroll
  for (int k = 0; k < kVec; ++k) {
    const float m2 = dec_f16(m232[k >> 1], k & 1) * m2_inv;
    const float w = dec_f16(w32[k >> 1], k & 1) * w_inv;
    out[k] = adam_update(g[k] * g_inv, m1[k] * m1_inv, m2, w, h);
  }
}

__device__ inline uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }

// the 8 updated elements of vector i encoded with the scales sc1 (m1,
// E4M3, saturating), sc2 (m2, FP16) and scw (w, FP16) and stored; the bf16
// copy of w too when w_bf16 is not null. Nontemporal stores: the state is
// streamed once per step (about 5 % faster than plain stores)
__device__ inline void store8(const Vals v[kVec], float sc1, float sc2, float scw, int64_t i, u32x2* m1, u32x4* m2,
                              u32x4* w, u32x4* w_bf16) {
  uint32_t q[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float f[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = fminf(fmaxf(v[4 * j + k].m1 * sc1, -448.0f), 448.0f);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], r, true);
    q[j] = (uint32_t)r;
  }
  __builtin_nontemporal_store((u32x2){q[0], q[1]}, m1 + i);
  uint32_t a[4], b[4], c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = enc_f16x2(v[2 * j].m2 * sc2, v[2 * j + 1].m2 * sc2);
    b[j] = enc_f16x2(v[2 * j].w * scw, v[2 * j + 1].w * scw);
    const f32x2 p = {v[2 * j].w, v[2 * j + 1].w};
    c[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
  }
  __builtin_nontemporal_store((u32x4){a[0], a[1], a[2], a[3]}, m2 + i);
  __builtin_nontemporal_store((u32x4){b[0], b[1], b[2], b[3]}, w + i);
  if (w_bf16) __builtin_nontemporal_store((u32x4){c[0], c[1], c[2], c[3]}, w_bf16 + i);
}

// the biases the step's new maxima give (m1: E4M3 rule, m2 and w: FP16
// rule), from the records' reduce_bits merged by the first pass
__device__ inline void new_biases(fp8_scale_t* s_m1, fp8_scale_t* s_m2, fp8_scale_t* s_w, int32_t b[3]) {
  b[0] = bias_from_amax_bits(__hip_atomic_load(&s_m1->reduce_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                             FP8_E4M3, 0, 0, nullptr);
  b[1] = bias_fp16_from_amax_bits(__hip_atomic_load(&s_m2->reduce_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                                  nullptr);
  b[2] = bias_fp16_from_amax_bits(__hip_atomic_load(&s_w->reduce_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                                  nullptr);
}

__device__ inline void block_merge_max(uint32_t v, uint32_t* target, uint32_t* lds) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = o > v ? o : v;
  }
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = lds[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) b = lds[i] > b ? lds[i] : b;
    const uint32_t seen = __hip_atomic_load(target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (b > seen) atomicMax(target, b);
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void adam_pass1_kernel(int64_t nvec, const u32x2* __restrict__ g8,
                                                              const fp8_scale_t* __restrict__ s_g,
                                                              const u32x2* __restrict__ m1,
                                                              fp8_scale_t* s_m1, const u32x4* __restrict__ m2,
                                                              fp8_scale_t* s_m2, const u32x4* __restrict__ w,
                                                              fp8_scale_t* s_w, AdamHyper h) {
  const float g_inv = s_g->scale_inv, m1_inv = s_m1->scale_inv, m2_inv = s_m2->scale_inv,
              w_inv = s_w->scale_inv;
  uint32_t x1 = 0, x2 = 0, xw = 0;  // fp32 magnitude bits; NaN sorts above inf
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * kThreads) {
    Vals v[kVec];
    update8(__builtin_nontemporal_load(g8 + i), __builtin_nontemporal_load(m1 + i),
            __builtin_nontemporal_load(m2 + i), __builtin_nontemporal_load(w + i), g_inv, m1_inv, m2_inv,
            w_inv, h, v);
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
      const uint32_t a = fbits(v[k].m1) & 0x7FFFFFFFu, b = fbits(v[k].m2) & 0x7FFFFFFFu,
                     c = fbits(v[k].w) & 0x7FFFFFFFu;
      x1 = a > x1 ? a : x1;
      x2 = b > x2 ? b : x2;
      xw = c > xw ? c : xw;
    }
  }
  __shared__ uint32_t lds[kThreads / 64];
  block_merge_max(x1, &s_m1->reduce_bits, lds);
  block_merge_max(x2, &s_m2->reduce_bits, lds);
  block_merge_max(xw, &s_w->reduce_bits, lds);
}

__global__ __launch_bounds__(kThreads) void adam_pass2_kernel(int64_t nvec, const u32x2* __restrict__ g8,
                                                              const fp8_scale_t* __restrict__ s_g, u32x2* m1,
                                                              fp8_scale_t* s_m1, u32x4* m2, fp8_scale_t* s_m2,
                                                              u32x4* w, fp8_scale_t* s_w, u32x4* w_bf16,
                                                              AdamHyper h) {
  const float g_inv = s_g->scale_inv, m1_inv = s_m1->scale_inv, m2_inv = s_m2->scale_inv,
              w_inv = s_w->scale_inv;
  int32_t b[3];
  new_biases(s_m1, s_m2, s_w, b);
  const float sc1 = pow2f(b[0]), sc2 = pow2f(b[1]), scw = pow2f(b[2]);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * kThreads) {
    Vals v[kVec];
    update8(g8[i], m1[i], m2[i], w[i], g_inv, m1_inv, m2_inv, w_inv, h, v);
    store8(v, sc1, sc2, scw, i, m1, m2, w, w_bf16);
  }
}

// One-pass variant, first kernel: the update of every element from the
// inputs, its maxima merged as in pass 1, and the new state encoded with
// the scales the records hold now (2^bias: a zeroed record's scale field
// reads 0, its bias 0) into the output buffers.
__global__ __launch_bounds__(kThreads) void adam_spec_kernel(int64_t nvec, const u32x2* __restrict__ g8,
                                                             const fp8_scale_t* __restrict__ s_g,
                                                             const u32x2* __restrict__ m1, const u32x4* __restrict__ m2,
                                                             const u32x4* __restrict__ w, u32x2* __restrict__ m1o,
                                                             u32x4* __restrict__ m2o, u32x4* __restrict__ wo,
                                                             fp8_scale_t* s_m1, fp8_scale_t* s_m2, fp8_scale_t* s_w,
                                                             u32x4* __restrict__ w_bf16, AdamHyper h) {
  const float g_inv = s_g->scale_inv, m1_inv = s_m1->scale_inv, m2_inv = s_m2->scale_inv,
              w_inv = s_w->scale_inv;
  const float sc1 = pow2f(s_m1->bias), sc2 = pow2f(s_m2->bias), scw = pow2f(s_w->bias);
  uint32_t x1 = 0, x2 = 0, xw = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * kThreads) {
    Vals v[kVec];
    update8(__builtin_nontemporal_load(g8 + i), __builtin_nontemporal_load(m1 + i),
            __builtin_nontemporal_load(m2 + i), __builtin_nontemporal_load(w + i), g_inv, m1_inv, m2_inv,
            w_inv, h, v);
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
      const uint32_t a = fbits(v[k].m1) & 0x7FFFFFFFu, b = fbits(v[k].m2) & 0x7FFFFFFFu,
                     c = fbits(v[k].w) & 0x7FFFFFFFu;
      x1 = a > x1 ? a : x1;
      x2 = b > x2 ? b : x2;
      xw = c > xw ? c : xw;
    }
    store8(v, sc1, sc2, scw, i, m1o, m2o, wo, w_bf16);
  }
  __shared__ uint32_t lds[kThreads / 64];
  block_merge_max(x1, &s_m1->reduce_bits, lds);
  block_merge_max(x2, &s_m2->reduce_bits, lds);
  block_merge_max(xw, &s_w->reduce_bits, lds);
}

// One-pass variant, second kernel: nothing to do when every new bias equals
// its record's (the common case: each block sees that and returns); else
// the whole update again from the untouched inputs, encoded with the new
// scales (the bf16 weights, the same fp32 values, were written already).
__global__ __launch_bounds__(kThreads) void adam_fix_kernel(int64_t nvec, const u32x2* __restrict__ g8,
                                                            const fp8_scale_t* __restrict__ s_g,
                                                            const u32x2* __restrict__ m1, const u32x4* __restrict__ m2,
                                                            const u32x4* __restrict__ w, u32x2* __restrict__ m1o,
                                                            u32x4* __restrict__ m2o, u32x4* __restrict__ wo,
                                                            fp8_scale_t* s_m1, fp8_scale_t* s_m2, fp8_scale_t* s_w,
                                                            AdamHyper h) {
  int32_t b[3];
  new_biases(s_m1, s_m2, s_w, b);
  if (b[0] == s_m1->bias && b[1] == s_m2->bias && b[2] == s_w->bias) return;
  const float g_inv = s_g->scale_inv, m1_inv = s_m1->scale_inv, m2_inv = s_m2->scale_inv,
              w_inv = s_w->scale_inv;
  const float sc1 = pow2f(b[0]), sc2 = pow2f(b[1]), scw = pow2f(b[2]);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * kThreads) {
    Vals v[kVec];
    update8(g8[i], m1[i], m2[i], w[i], g_inv, m1_inv, m2_inv, w_inv, h, v);
    store8(v, sc1, sc2, scw, i, m1o, m2o, wo, nullptr);
  }
}

// missed (or null): bit i set where record i (m1, m2, w) changed its bias
__global__ void adam_publish_kernel(fp8_scale_t* s_m1, fp8_scale_t* s_m2, fp8_scale_t* s_w, uint32_t* missed) {
  fp8_scale_t* recs[3] = {s_m1, s_m2, s_w};
  uint32_t changed = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    fp8_scale_t* s = recs[i];
    const uint32_t mag = s->reduce_bits;
    uint32_t flags;
    const int32_t b = i == 0 ? bias_from_amax_bits(mag, FP8_E4M3, 0, 0, &flags) : bias_fp16_from_amax_bits(mag, &flags);
    if (b != s->bias) changed |= 1u << i;
    s->amax = __builtin_bit_cast(float, mag);
    s->bias = b;
    s->scale = pow2f(b);
    s->scale_inv = pow2f(-b);
    s->flags = flags;
    s->reduce_bits = 0u;
  }
  if (missed) *missed = changed;
}

// master-weight initialisation: bf16 weights -> FP16 with a per-tensor scale
__global__ __launch_bounds__(kThreads) void master_amax_kernel(int64_t nvec, const u32x4* __restrict__ src,
                                                               fp8_scale_t* s_w) {
  uint32_t x = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * kThreads) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = (u[k] & 0x7FFFu) << 16, hi = u[k] & 0x7FFF0000u;
      x = lo > x ? lo : x;
      x = hi > x ? hi : x;
    }
  }
  __shared__ uint32_t lds[kThreads / 64];
  block_merge_max(x, &s_w->reduce_bits, lds);
}

__global__ __launch_bounds__(kThreads) void master_encode_kernel(int64_t nvec, const u32x4* __restrict__ src,
                                                                 u32x4* __restrict__ w, fp8_scale_t* s_w) {
  const uint32_t mag = __hip_atomic_load(&s_w->reduce_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float sc = pow2f(bias_fp16_from_amax_bits(mag, nullptr));
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * kThreads) {
    const u32x4 v = src[i];
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = enc_f16x2(__builtin_bit_cast(float, u[k] << 16) * sc, __builtin_bit_cast(float, u[k] & 0xFFFF0000u) * sc);
    w[i] = (u32x4){o[0], o[1], o[2], o[3]};
  }
}

__global__ void master_publish_kernel(fp8_scale_t* s_w) {
  const uint32_t mag = s_w->reduce_bits;
  uint32_t flags;
  const int32_t b = bias_fp16_from_amax_bits(mag, &flags);
  s_w->amax = __builtin_bit_cast(float, mag);
  s_w->bias = b;
  s_w->scale = pow2f(b);
  s_w->scale_inv = pow2f(-b);
  s_w->flags = flags;
  s_w->reduce_bits = 0u;
}

int64_t grid_for(int64_t nvec) {
  int64_t blocks = (nvec + kThreads - 1) / kThreads;
  return blocks < 1 ? 1 : (blocks > kMaxBlocks ? kMaxBlocks : blocks);
}

}  // namespace

hipError_t launch_master_init(int64_t n, const uint16_t* w_bf16, uint16_t* w, fp8_scale_t* s_w, hipStream_t st) {
  const int64_t nvec = n / 8;  // 8 bf16 per 16 bytes
  const unsigned blocks = (unsigned)grid_for(nvec);
  hipLaunchKernelGGL(master_amax_kernel, dim3(blocks), dim3(kThreads), 0, st, nvec, (const u32x4*)w_bf16, s_w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(master_encode_kernel, dim3(blocks), dim3(kThreads), 0, st, nvec, (const u32x4*)w_bf16,
                     (u32x4*)w, s_w);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(master_publish_kernel, dim3(1), dim3(1), 0, st, s_w);
  return hipGetLastError();
}

hipError_t launch_adam(int64_t n, const uint8_t* g8, const fp8_scale_t* s_g, uint8_t* m1, fp8_scale_t* s_m1,
                       uint16_t* m2, fp8_scale_t* s_m2, uint16_t* w, fp8_scale_t* s_w, uint16_t* w_bf16,
                       const AdamHyper& h, hipStream_t st) {
  const int64_t nvec = n / kVec;
  const int64_t blocks = grid_for(nvec);
  hipLaunchKernelGGL(adam_pass1_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, nvec, (const u32x2*)g8, s_g,
                     (const u32x2*)m1, s_m1, (const u32x4*)m2, s_m2, (const u32x4*)w, s_w, h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(adam_pass2_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, nvec, (const u32x2*)g8, s_g,
                     (u32x2*)m1, s_m1, (u32x4*)m2, s_m2, (u32x4*)w, s_w, (u32x4*)w_bf16, h);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(adam_publish_kernel, dim3(1), dim3(1), 0, st, s_m1, s_m2, s_w, (uint32_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_adam_spec(int64_t n, const uint8_t* g8, const fp8_scale_t* s_g, const uint8_t* m1,
                            const uint16_t* m2, const uint16_t* w, uint8_t* m1_out, uint16_t* m2_out, uint16_t* w_out,
                            fp8_scale_t* s_m1, fp8_scale_t* s_m2, fp8_scale_t* s_w, uint16_t* w_bf16,
                            uint32_t* missed, const AdamHyper& h, hipStream_t st) {
  const int64_t nvec = n / kVec;
  const int64_t blocks = grid_for(nvec);
  hipLaunchKernelGGL(adam_spec_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, nvec, (const u32x2*)g8, s_g,
                     (const u32x2*)m1, (const u32x4*)m2, (const u32x4*)w, (u32x2*)m1_out, (u32x4*)m2_out,
                     (u32x4*)w_out, s_m1, s_m2, s_w, (u32x4*)w_bf16, h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(adam_fix_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, nvec, (const u32x2*)g8, s_g,
                     (const u32x2*)m1, (const u32x4*)m2, (const u32x4*)w, (u32x2*)m1_out, (u32x4*)m2_out,
                     (u32x4*)w_out, s_m1, s_m2, s_w, h);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(adam_publish_kernel, dim3(1), dim3(1), 0, st, s_m1, s_m2, s_w, missed);
  return hipGetLastError();
}

}  // namespace fp8lin
