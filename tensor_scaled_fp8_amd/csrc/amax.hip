// a1 amax (+ a2 scale choice) over a bf16 tensor.
//
// [Perez et al. review, "Proposed method", bullets 1-2] the scaling bias of
// a tensor comes from its max |x|. One pass over HBM with 16-byte
// nontemporal loads (streamed past the caches, which keeps reads near the
// HBM rate). |x| is compared on the 15-bit magnitude pattern: for bf16,
// the integer order of (bits & 0x7FFF) is the order of |x|, with inf above
// every finite value and NaN patterns above inf, so the integer max also
// detects non-finite values. Two packed 16-bit maxima per dword (one VALU
// op per two values), a wavefront max by cross-lane exchange, a block max
// through LDS. Blocks then merge (tag << 16) | max into the record's 64-bit
// gen_max word with a device-scope atomic max, skipped when the word
// already holds at least as much (same-address atomics from many blocks
// serialise); tag = the record's epoch + 1 and the consumer of the maximum
// advances epoch, so older maxima never win, nothing waits inside the
// kernel and the word is never cleared. What follows on the stream reads
// the word and advances epoch:
//  * fp8_amax / fp8_amax_scale: a one-thread kernel publishes amax (and the
//    scale). A last-block ticket in the reduction kernel itself was
//    measured 6-8 us slower per call: every block has to wait for its merge
//    and then for a same-address counter, which serialises 512 blocks.
//  * fp8_quantize: the cast kernel derives the scale from the word and
//    publishes the record.
#include "fp8lin_internal.h"

namespace fp8lin {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;        // 16-byte loads in flight per thread
// 1.5 blocks per CU on 256 CUs (one merge atomic each at most): the best of
// 256 / 384 / 512 / 1024 / 2048 on 32-128 MB tensors; more blocks end with
// more merges on the one word and measured slower
constexpr int kMaxBlocks = 384;

__device__ inline u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }

__device__ inline u16x2 vmax(u16x2 a, uint32_t w) {
  return __builtin_elementwise_max(a, as_u16x2(w & 0x7FFF7FFFu));
}

__device__ inline void write_scale(fp8_scale_t* s, uint32_t mag, bool fuse, int fmt, int margin,
                                   int mu_log2) {
  union { uint32_t u; float f; } a;
  a.u = mag << 16;
  uint32_t flags = 0;
  int32_t b = 0;
  if (fuse) {
    b = bias_from_amax_bits(mag << 16, fmt, margin, mu_log2, &flags);
  } else {
    flags = mag >= 0x7F80u ? FP8_FLAG_NONFINITE : (mag == 0u ? FP8_FLAG_ZERO : 0u);
  }
  s->amax = a.f;
  s->bias = b;
  s->scale = pow2f(b);
  s->scale_inv = pow2f(-b);
  s->flags = flags;
}

// Block-wide max of |x| bits over chunk blk of the tensor (block-
// contiguous chunks of whole kUnroll*256-vector steps; chunk 0 also takes
// the < 8-element tail). The result is valid in thread 0.
__device__ inline uint32_t block_max_bits(const u32x4* __restrict__ x, int64_t n_vec, int64_t per_block,
                                          const uint16_t* __restrict__ tail, int tail_n, int blk) {
  u16x2 m = {0, 0};
  const int64_t b0 = (int64_t)blk * per_block;
  const int64_t b1 = b0 + per_block < n_vec ? b0 + per_block : n_vec;
  int64_t base = b0;
  for (; base + kUnroll * kThreads <= b1; base += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(x + base + u * kThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      m = vmax(m, v[u].x);
      m = vmax(m, v[u].y);
      m = vmax(m, v[u].z);
      m = vmax(m, v[u].w);
    }
  }
  for (int64_t i = base + threadIdx.x; i < b1; i += kThreads) {
    const u32x4 v = __builtin_nontemporal_load(x + i);
    m = vmax(m, v.x);
    m = vmax(m, v.y);
    m = vmax(m, v.z);
    m = vmax(m, v.w);
  }
  if (blk == 0 && (int)threadIdx.x < tail_n) {
    m = vmax(m, (uint32_t)tail[threadIdx.x]);
  }
  uint32_t r = m.x > m.y ? m.x : m.y;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {  // wavefront max
    uint32_t o = (uint32_t)__shfl_xor((int)r, off, 64);
    r = o > r ? o : r;
  }
  __shared__ uint32_t wmax[kThreads / 64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) wmax[wid] = r;
  __syncthreads();
  uint32_t b = wmax[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) b = wmax[w] > b ? wmax[w] : b;
  return b;
}

// merge (tag << 16) | b into the record's tagged maximum (see above)
__device__ inline void merge_max(fp8_scale_t* s, uint32_t b) {
  const unsigned long long v = (reduction_tag(s) << 16) | b;
  unsigned long long* word = (unsigned long long*)&s->gen_max;
  const unsigned long long seen = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (v > seen) atomicMax(word, v);
}

__global__ __launch_bounds__(kThreads) void amax_gen_kernel(const u32x4* __restrict__ x, int64_t n_vec,
                                                            int64_t per_block,
                                                            const uint16_t* __restrict__ tail,
                                                            int tail_n, fp8_scale_t* s) {
  const uint32_t b = block_max_bits(x, n_vec, per_block, tail, tail_n, (int)blockIdx.x);
  if (threadIdx.x == 0) merge_max(s, b);
}

// amax passes of up to kQuantBatchMax tensors in one launch: blocks
// first_block[i] .. first_block[i+1]-1 sweep tensor i's chunks and merge
// into its record, exactly as amax_gen_kernel's blocks would.
struct AmaxEntry {
  const u32x4* x;
  int64_t n_vec, per_block;
  const uint16_t* tail;
  fp8_scale_t* s;
  int tail_n, first_block;
};
struct AmaxBatch {
  AmaxEntry e[kQuantBatchMax];
  int count;
};

__global__ __launch_bounds__(kThreads) void amax_batch_kernel(AmaxBatch bt) {
  const int blk = (int)blockIdx.x;
  int i = 0;
#pragma unroll
  for (int k = 1; k < kQuantBatchMax; ++k)
    if (k < bt.count && blk >= bt.e[k].first_block) i = k;
  const AmaxEntry& e = bt.e[i];
  const uint32_t b = block_max_bits(e.x, e.n_vec, e.per_block, e.tail, e.tail_n, blk - e.first_block);
  if (threadIdx.x == 0) merge_max(e.s, b);
}

// fp8_amax / fp8_amax_scale: publish the maximum the reduction just merged
// (the low 16 bits of gen_max, whose tag is this call's) and advance epoch
__global__ void amax_publish_kernel(fp8_scale_t* s, int fuse, int fmt, int margin, int mu_log2) {
  const unsigned long long word =
      __hip_atomic_load((unsigned long long*)&s->gen_max, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  write_scale(s, (uint32_t)(word & 0xFFFFu), fuse != 0, fmt, margin, mu_log2);
  s->epoch = word >> 16;
}

__global__ void scale_kernel(fp8_scale_t* s, int fmt, int margin, int mu_log2) {
  union { float f; uint32_t u; } a;
  a.f = s->amax;
  uint32_t flags;
  int32_t b = bias_from_amax_bits(a.u & 0x7FFFFFFFu, fmt, margin, mu_log2, &flags);
  s->bias = b;
  s->scale = pow2f(b);
  s->scale_inv = pow2f(-b);
  s->flags = flags;
}

// FP8-CSCALE: a constant bias instead of the amax rule; the internal words
// are left alone so the record stays usable by the amax paths
__global__ void scale_fixed_kernel(fp8_scale_t* s, int32_t b) {
  s->amax = 0.0f;
  s->bias = b;
  s->scale = pow2f(b);
  s->scale_inv = pow2f(-b);
  s->flags = 0u;
}

__global__ void scale_reset_kernel(uint4* s, int64_t n16) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) s[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_scale_reset(fp8_scale_t* s, int64_t count, hipStream_t st) {
  if (count == 0) return hipSuccess;
  const int64_t n16 = count * (int64_t)(sizeof(fp8_scale_t) / 16);
  const int64_t blocks = (n16 + 255) / 256;
  hipLaunchKernelGGL(scale_reset_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (uint4*)s, n16);
  return hipGetLastError();
}

namespace {
struct SweepGrid {
  int64_t n_vec, per_block, blocks;
  int tail_n;
  const uint16_t* tail;
};
// enough blocks to fill the chip (at most max_blocks), each a contiguous
// chunk of whole steps
SweepGrid sweep_grid(const void* x, int64_t n, int64_t max_blocks = kMaxBlocks) {
  SweepGrid g;
  g.n_vec = n / 8;
  g.tail_n = (int)(n - g.n_vec * 8);
  g.tail = (const uint16_t*)x + g.n_vec * 8;
  const int64_t step = (int64_t)kThreads * kUnroll;
  int64_t blocks = (g.n_vec + step - 1) / step;
  blocks = blocks < 1 ? 1 : (blocks > max_blocks ? max_blocks : blocks);
  g.per_block = ((g.n_vec + blocks - 1) / blocks + step - 1) / step * step;
  g.blocks = g.n_vec > 0 ? (g.n_vec + g.per_block - 1) / g.per_block : 1;
  return g;
}
}  // namespace

hipError_t launch_amax_gen(const void* x, int64_t n, fp8_scale_t* s, hipStream_t st) {
  const SweepGrid g = sweep_grid(x, n);
  hipLaunchKernelGGL(amax_gen_kernel, dim3((unsigned)g.blocks), dim3(kThreads), 0, st, (const u32x4*)x,
                     g.n_vec, g.per_block, g.tail, g.tail_n, s);
  return hipGetLastError();
}

hipError_t launch_amax_batch(const QuantDesc* d, int count, hipStream_t st) {
  if (count < 1 || count > kQuantBatchMax) return hipErrorInvalidValue;
  // the chip-filling block budget of one sweep, shared in proportion to size
  int64_t total = 0;
  for (int i = 0; i < count; ++i) total += d[i].rows * d[i].cols;
  AmaxBatch bt{};
  bt.count = count;
  int blocks = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t n = d[i].rows * d[i].cols;
    const int64_t cap = total > 0 ? (kMaxBlocks * n + total - 1) / total : 1;
    const SweepGrid g = sweep_grid(d[i].x, n, cap < 1 ? 1 : cap);
    AmaxEntry& e = bt.e[i];
    e.x = (const u32x4*)d[i].x;
    e.n_vec = g.n_vec;
    e.per_block = g.per_block;
    e.tail = g.tail;
    e.tail_n = g.tail_n;
    e.s = d[i].s;
    e.first_block = blocks;
    blocks += (int)g.blocks;
  }
  hipLaunchKernelGGL(amax_batch_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, bt);
  return hipGetLastError();
}

hipError_t launch_amax(const void* x, int64_t n, fp8_scale_t* s, bool fuse_scale, int fmt, int margin,
                       int mu_log2, hipStream_t st) {
  const hipError_t e = launch_amax_gen(x, n, s, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(amax_publish_kernel, dim3(1), dim3(1), 0, st, s, fuse_scale ? 1 : 0, fmt, margin, mu_log2);
  return hipGetLastError();
}

hipError_t launch_scale_fixed(fp8_scale_t* s, int32_t bias, hipStream_t st) {
  hipLaunchKernelGGL(scale_fixed_kernel, dim3(1), dim3(1), 0, st, s, bias);
  return hipGetLastError();
}

hipError_t launch_scale(fp8_scale_t* s, int fmt, int margin, int mu_log2, hipStream_t st) {
  hipLaunchKernelGGL(scale_kernel, dim3(1), dim3(1), 0, st, s, fmt, margin, mu_log2);
  return hipGetLastError();
}

}  // namespace fp8lin
