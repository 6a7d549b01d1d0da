// a3 cast (+ transpose): bf16 [rows, cols] -> FP8 codes, row-wise [rows, cols]
// and transposed [cols, rows].
//
// [Perez et al. review, "Proposed method", bullets 3-4] the tensor is
// multiplied by its scale 2^bias before the FP8 cast (E4M3 for weights and
// activations, E5M2 for gradients). The product is exact (a power of two);
// it is clamped to +-max (saturation; inf -> max) and converted by the
// hardware FP8 converter, which rounds to nearest even and keeps
// subnormals. NaN inputs are patched to 0x7F|sign afterwards: with a
// derived scale only where the record's FP8_FLAG_NONFINITE says the tensor
// holds one; with a published record (e.g. a fixed bias, whose record says
// nothing about the tensor) wherever a thread's patch holds one.
//
// Inputs are read with nontemporal loads (streamed past the caches).
// Tiling: one 256-thread block per 128 x 128 tile. Each thread loads an
// 8 x 8 patch (eight 16-byte row loads), converts it, stores its eight
// 8-byte row-wise pieces, transposes the 8 x 8 bytes in registers
// (byte permutes) and writes eight 8-byte column pieces into an LDS tile
// laid out transposed. After a barrier the block streams the transposed
// tile out as 16-byte stores, 128 contiguous bytes per output row, so both
// outputs are written in whole 128-byte lines. LDS chunks are XOR-swizzled
// by (row / 8) so the 8-byte column writes spread over the banks.
//
// Also here: the casts of several tensors in one launch (cast_batch_kernel,
// fp8_quantize_batch), and the speculative one-pass quantise
// (quantize_spec_kernel casting with the record's previous bias while
// taking the amax, quantize_check_kernel recasting only if the bias
// changed; fp8_quantize_spec).
#include "fp8lin_internal.h"

namespace fp8lin {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 128;
constexpr int kThreads = 256;
constexpr int64_t kSpecBlocks = 512;  // grid cap of the speculative quantise (one merge per block)
constexpr int kSpecGroups = 4;        // 256-thread tile groups per speculative block
constexpr int kSpecTiles = 2;         // tiles whose loads one group step keeps in flight

template <int FMT>
__device__ inline uint32_t cvt4(uint32_t w0, uint32_t w1, float scale) {
  constexpr float kMax = FMT == FP8_E4M3 ? 448.0f : 57344.0f;
  float f0 = __uint_as_float(w0 << 16) * scale;
  float f1 = __uint_as_float(w0 & 0xFFFF0000u) * scale;
  float f2 = __uint_as_float(w1 << 16) * scale;
  float f3 = __uint_as_float(w1 & 0xFFFF0000u) * scale;
  f0 = fminf(fmaxf(f0, -kMax), kMax);
  f1 = fminf(fmaxf(f1, -kMax), kMax);
  f2 = fminf(fmaxf(f2, -kMax), kMax);
  f3 = fminf(fmaxf(f3, -kMax), kMax);
  int r;
  if constexpr (FMT == FP8_E4M3) {
    r = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, r, true);
  } else {
    r = __builtin_amdgcn_cvt_pk_bf8_f32(f0, f1, 0, false);
    r = __builtin_amdgcn_cvt_pk_bf8_f32(f2, f3, r, true);
  }
  return (uint32_t)r;
}

// NaN bf16 inputs -> 0x7F with the input's sign, byte by byte.
__device__ inline uint32_t patch_nan(uint32_t q, uint32_t w0, uint32_t w1) {
  const uint32_t h[4] = {w0 & 0xFFFFu, w0 >> 16, w1 & 0xFFFFu, w1 >> 16};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if ((h[k] & 0x7FFFu) > 0x7F80u) {
      const uint32_t code = 0x7Fu | ((h[k] >> 8) & 0x80u);
      q = (q & ~(0xFFu << (8 * k))) | (code << (8 * k));
    }
  }
  return q;
}

// 4 x 4 byte transpose: in[i] holds row i (bytes = cols 0..3); out[j] holds
// column j (bytes = rows 0..3).
__device__ inline void transpose4(const uint32_t in[4], uint32_t out[4]) {
  const uint32_t a0 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);  // r0c0 r1c0 r0c1 r1c1
  const uint32_t a1 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);  // r0c2 r1c2 r0c3 r1c3
  const uint32_t b0 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);  // r2c0 r3c0 r2c1 r3c1
  const uint32_t b1 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(b0, a0, 0x05040100u);  // r0c0 r1c0 r2c0 r3c0
  out[1] = __builtin_amdgcn_perm(b0, a0, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(b1, a1, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(b1, a1, 0x07060302u);
}

// The tagged maximum the reduction before this kernel merged. It is final
// while this kernel runs (only a later reduction changes it), so a plain
// load of the uniform address does: one request per wave, where a
// device-scope atomic load per thread (a thousand blocks of 256 threads on
// one address) measured ~3 us per launch.
__device__ inline unsigned long long merged_max(const fp8_scale_t* s) { return s->gen_max; }

// LDS of a cast block, declared once for the file so that a kernel holding
// both format variants (the batch kernel) still needs only this much.
__shared__ uint4 g_tile[kTile * kTile / 16];  // transposed tile: 128 rows of 128 bytes
__shared__ uint32_t g_wsum[kThreads / 64];    // COUNT: per-wave sums

// DERIVE = false: the scale comes from the record's published fields.
// DERIVE = true (fp8_quantize): every block derives it from the record's
// tagged maximum, which the amax pass just merged, with the same rule as
// fp8_scale; block 0 publishes the record's fields and advances its epoch
// to the tag it consumed.
// COUNT (with DERIVE): also count the elements whose scaled magnitude
// exceeds the format's max (inf included, NaN not) into s->sat_count, which
// the kernel before this one cleared.
// tile: index of the 128 x 128 tile within the tensor (row-major over tiles).
template <int FMT, bool DERIVE, bool COUNT>
__device__ __forceinline__ void cast_tile(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                          int64_t tiles_c, fp8_scale_t* s, uint8_t* __restrict__ out_row,
                                          uint8_t* __restrict__ out_t, int margin, int mu_log2, int64_t tile) {
  uint4* const lds = g_tile;
  const int t = threadIdx.x;
  const int64_t tr = tile / tiles_c, tc = tile - (tile / tiles_c) * tiles_c;
  const int64_t r0 = tr * kTile, c0 = tc * kTile;
  const int rg = t >> 4, cc = t & 15;
  float scale;
  bool nonfinite;
  uint32_t sat_above = 0x7F80u;  // COUNT: magnitudes above this (and <= inf) saturate
  if constexpr (DERIVE) {
    const unsigned long long word = merged_max(s);
    const uint32_t mag = (uint32_t)(word & 0xFFFFu);
    uint32_t flags;
    const int32_t b = bias_from_amax_bits(mag << 16, FMT, margin, mu_log2, &flags);
    scale = pow2f(b);
    if constexpr (COUNT) {
      // fmt max = 1.75 * 2^E; max * 2^-b as a bf16 pattern: exponent field
      // 127 + E - b, mantissa 0x60; beyond the bf16 range no finite value
      // saturates
      const int e = 127 + (FMT == FP8_E4M3 ? 8 : 15) - b;
      sat_above = e <= 254 ? (((uint32_t)e << 7) | 0x60u) : 0x7F7Fu;
    }
    nonfinite = (flags & FP8_FLAG_NONFINITE) != 0u;
    if (tile == 0 && t == 0) {
      union { uint32_t u; float f; } a;
      a.u = mag << 16;
      s->amax = a.f;
      s->bias = b;
      s->scale = scale;
      s->scale_inv = pow2f(-b);
      s->flags = flags;
      s->epoch = word >> 16;  // this call's maximum is consumed
    }
  } else {
    // a published record need not describe this tensor (fp8_scale_fixed
    // writes no flags): NaNs are looked for in each patch below
    scale = s->scale;
    nonfinite = false;
  }
  const int64_t rr = r0 + 8 * rg, cx = c0 + 8 * cc;
  const bool ok = rr < rows && cx < cols;  // rows, cols are multiples of 16

  uint32_t lo[8], hi[8];
  uint32_t nsat = 0;
  if (ok) {
    const uint16_t* src = x + rr * cols + cx;
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __builtin_nontemporal_load((const u32x4*)(src + i * cols));
    if constexpr (COUNT) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t a = w4[k] & 0x7FFFu, b2 = (w4[k] >> 16) & 0x7FFFu;
          nsat += (a > sat_above && a <= 0x7F80u) + (b2 > sat_above && b2 <= 0x7F80u);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo[i] = cvt4<FMT>(v[i].x, v[i].y, scale);
      hi[i] = cvt4<FMT>(v[i].z, v[i].w, scale);
    }
    if constexpr (!DERIVE) {
      // any NaN (magnitude bits above 0x7F80) in this thread's patch
      u16x2 m = {0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, (uint32_t)(v[i].x & 0x7FFF7FFFu)));
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, (uint32_t)(v[i].y & 0x7FFF7FFFu)));
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, (uint32_t)(v[i].z & 0x7FFF7FFFu)));
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, (uint32_t)(v[i].w & 0x7FFF7FFFu)));
      }
      nonfinite = (m.x > m.y ? m.x : m.y) > 0x7F80u;
    }
    if (nonfinite) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo[i] = patch_nan(lo[i], v[i].x, v[i].y);
        hi[i] = patch_nan(hi[i], v[i].z, v[i].w);
      }
    }
    if (out_row) {
      uint8_t* dst = out_row + rr * cols + cx;
#pragma unroll
      for (int i = 0; i < 8; ++i) *(uint2*)(dst + i * cols) = make_uint2(lo[i], hi[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) lo[i] = hi[i] = 0u;
  }
  if constexpr (COUNT) {
    // an empty tensor has no producer kernel that cleared the count
    if ((rows == 0 || cols == 0) && t == 0) s->sat_count = 0u;
    // block sum, one atomic per block that saw a saturation
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) nsat += (uint32_t)__shfl_xor((int)nsat, off, 64);
    uint32_t* const wsum = g_wsum;
    if ((t & 63) == 0) wsum[t >> 6] = nsat;
    __syncthreads();
    if (t == 0) {
      uint32_t tot = 0;
#pragma unroll
      for (int i = 0; i < kThreads / 64; ++i) tot += wsum[i];
      if (tot) atomicAdd(&s->sat_count, tot);
    }
  }
  if (!out_t) return;

  // column j of the patch: rows 0-3 in c03[j], rows 4-7 in c47[j]
  uint32_t c03[8], c47[8];
  transpose4(&lo[0], &c03[0]);
  transpose4(&hi[0], &c03[4]);
  transpose4(&lo[4], &c47[0]);
  transpose4(&hi[4], &c47[4]);
  uint8_t* l8 = (uint8_t*)lds;
  const int sw = cc & 7;  // = (transposed row / 8) & 7
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int trow = 8 * cc + j;
    const int off = trow * kTile + ((((rg >> 1) ^ sw)) << 4) + 8 * (rg & 1);
    *(uint2*)(l8 + off) = make_uint2(c03[j], c47[j]);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int q = t + kThreads * k;
    const int trow = q >> 3, part = q & 7;
    const uint4 v = lds[trow * 8 + (part ^ ((trow >> 3) & 7))];
    const int64_t oc = c0 + trow, orow = r0 + 16 * part;
    if (oc < cols && orow < rows) *(uint4*)(out_t + oc * rows + orow) = v;
  }
}

template <int FMT, bool DERIVE, bool COUNT = false>
__global__ __launch_bounds__(kThreads) void cast_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                        int64_t cols, int64_t tiles_c, fp8_scale_t* s,
                                                        uint8_t* __restrict__ out_row,
                                                        uint8_t* __restrict__ out_t, int margin,
                                                        int mu_log2) {
  cast_tile<FMT, DERIVE, COUNT>(x, rows, cols, tiles_c, s, out_row, out_t, margin, mu_log2, (int64_t)blockIdx.x);
}

// Derive-casts of up to kQuantBatchMax tensors in one launch: blocks
// first_block[i] .. first_block[i+1]-1 take tensor i's tiles (an empty
// tensor gets one block, which publishes its record). Each block does what
// fp8_quantize's cast block for that tile does.
struct CastEntry {
  const uint16_t* x;
  int64_t rows, cols, tiles_c;
  fp8_scale_t* s;
  uint8_t* out_row;
  uint8_t* out_t;
  int fmt, margin, mu_log2, first_block;
};
struct CastBatch {
  CastEntry e[kQuantBatchMax];
  int count;
};

__global__ __launch_bounds__(kThreads) void cast_batch_kernel(CastBatch b) {
  const int blk = (int)blockIdx.x;
  int i = 0;
#pragma unroll
  for (int k = 1; k < kQuantBatchMax; ++k)
    if (k < b.count && blk >= b.e[k].first_block) i = k;
  const CastEntry& e = b.e[i];
  const int64_t tile = blk - e.first_block;
  if (e.fmt == FP8_E4M3)
    cast_tile<FP8_E4M3, true, false>(e.x, e.rows, e.cols, e.tiles_c, e.s, e.out_row, e.out_t, e.margin, e.mu_log2,
                                     tile);
  else
    cast_tile<FP8_E5M2, true, false>(e.x, e.rows, e.cols, e.tiles_c, e.s, e.out_row, e.out_t, e.margin, e.mu_log2,
                                     tile);
}

// Speculative a1 + a3 in one pass: each block casts its tiles (tile
// blockIdx.x, then every gridDim.x-th, kSpecTiles at a time) with the bias the record holds from
// its previous quantisation (the guess; block 0 keeps it in s->spec_bias),
// and merges the max |x| of its tiles into the tagged maximum as the amax
// pass does (one merge per block, so the grid stays small). NaN bytes are
// patched where a thread's patch holds a NaN (the same bytes the
// derive-cast writes); +-inf and out-of-range values saturate, as there.
template <int FMT>
__global__ __launch_bounds__(kThreads * kSpecGroups) void quantize_spec_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t tiles_c, int64_t ntiles, fp8_scale_t* s,
    uint8_t* __restrict__ out_row) {
  const int t = threadIdx.x;
  const int rg = (t & (kThreads - 1)) >> 4, cc = t & 15;
  const int32_t guess = s->bias;
  const float scale = pow2f(guess);
  uint32_t mag = 0;
  // each 256-thread group takes kSpecTiles tiles per step (tiles g, g + G,
  // ..., G = the grid's group count) and issues all their loads before it
  // converts any; four groups per block keep many waves resident per CU
  // while the number of blocks, and so of merges, stays small
  const int64_t G = (int64_t)gridDim.x * kSpecGroups;
  for (int64_t base = (int64_t)blockIdx.x * kSpecGroups + (t >> 8); base < ntiles; base += kSpecTiles * G) {
    u32x4 v[kSpecTiles][8];
    int64_t off[kSpecTiles];
    bool ok[kSpecTiles];
#pragma unroll
    for (int j = 0; j < kSpecTiles; ++j) {
      const int64_t tile = base + j * G;
      const int64_t tr = tile / tiles_c, tc = tile - (tile / tiles_c) * tiles_c;
      const int64_t rr = tr * kTile + 8 * rg, cx = tc * kTile + 8 * cc;
      ok[j] = tile < ntiles && rr < rows && cx < cols;
      off[j] = rr * cols + cx;
      if (ok[j]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[j][i] = __builtin_nontemporal_load((const u32x4*)(x + off[j] + i * cols));
      }
    }
#pragma unroll
    for (int j = 0; j < kSpecTiles; ++j) {
      if (!ok[j]) continue;
      u16x2 m = {0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, (uint32_t)(v[j][i].x & 0x7FFF7FFFu)));
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, (uint32_t)(v[j][i].y & 0x7FFF7FFFu)));
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, (uint32_t)(v[j][i].z & 0x7FFF7FFFu)));
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, (uint32_t)(v[j][i].w & 0x7FFF7FFFu)));
      }
      const uint32_t tmag = m.x > m.y ? m.x : m.y;
      mag = tmag > mag ? tmag : mag;
      uint32_t lo[8], hi[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo[i] = cvt4<FMT>(v[j][i].x, v[j][i].y, scale);
        hi[i] = cvt4<FMT>(v[j][i].z, v[j][i].w, scale);
      }
      if (tmag > 0x7F80u) {  // a NaN in this thread's patch
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          lo[i] = patch_nan(lo[i], v[j][i].x, v[j][i].y);
          hi[i] = patch_nan(hi[i], v[j][i].z, v[j][i].w);
        }
      }
      uint8_t* dst = out_row + off[j];
#pragma unroll
      for (int i = 0; i < 8; ++i) *(uint2*)(dst + i * cols) = make_uint2(lo[i], hi[i]);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {  // wavefront max
    const uint32_t o = (uint32_t)__shfl_xor((int)mag, off, 64);
    mag = o > mag ? o : mag;
  }
  __shared__ uint32_t wmax[kThreads * kSpecGroups / 64];
  if ((t & 63) == 0) wmax[t >> 6] = mag;
  __syncthreads();
  if (t == 0) {
    uint32_t b = wmax[0];
#pragma unroll
    for (int i = 1; i < kThreads * kSpecGroups / 64; ++i) b = wmax[i] > b ? wmax[i] : b;
    const unsigned long long val = (reduction_tag(s) << 16) | b;
    unsigned long long* word = (unsigned long long*)&s->gen_max;
    const unsigned long long seen = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (val > seen) atomicMax(word, val);
    if (blockIdx.x == 0) s->spec_bias = guess;
  }
}

// The check after quantize_spec_kernel: the bias from the merged maximum
// (the rule of fp8_quantize); block 0 publishes the record. Where it equals
// the guess the speculative bytes are final; otherwise every block recasts
// its tile with it (the derive-cast tile body).
template <int FMT>
__global__ __launch_bounds__(kThreads) void quantize_check_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                  int64_t cols, int64_t tiles_c, int64_t ntiles,
                                                                  fp8_scale_t* s, uint8_t* __restrict__ out_row,
                                                                  int margin, int mu_log2) {
  const unsigned long long word = merged_max(s);
  uint32_t flags;
  const int32_t b = bias_from_amax_bits((uint32_t)(word & 0xFFFFu) << 16, FMT, margin, mu_log2, &flags);
  if (b == s->spec_bias) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      union { uint32_t u; float f; } a;
      a.u = (uint32_t)(word & 0xFFFFu) << 16;
      s->amax = a.f;
      s->bias = b;
      s->scale = pow2f(b);
      s->scale_inv = pow2f(-b);
      s->flags = flags;
      s->epoch = word >> 16;
    }
    return;
  }
  // recast (the block holding tile 0 publishes the same record fields inside)
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x)
    cast_tile<FMT, true, false>(x, rows, cols, tiles_c, s, out_row, nullptr, margin, mu_log2, tile);
}

template <bool DERIVE, bool COUNT = false>
hipError_t launch_cast_t(const void* x, int64_t rows, int64_t cols, int fmt, fp8_scale_t* s,
                         uint8_t* out_row, uint8_t* out_t, int margin, int mu_log2, hipStream_t st) {
  int64_t tiles_r = (rows + kTile - 1) / kTile, tiles_c = (cols + kTile - 1) / kTile;
  if (tiles_r * tiles_c == 0) tiles_r = tiles_c = 1;  // empty: one block that reads nothing (publishes)
  const dim3 grid((unsigned)(tiles_r * tiles_c));
  if (fmt == FP8_E4M3)
    hipLaunchKernelGGL((cast_kernel<FP8_E4M3, DERIVE, COUNT>), grid, dim3(kThreads), 0, st,
                       (const uint16_t*)x, rows, cols, tiles_c, s, out_row, out_t, margin, mu_log2);
  else
    hipLaunchKernelGGL((cast_kernel<FP8_E5M2, DERIVE, COUNT>), grid, dim3(kThreads), 0, st,
                       (const uint16_t*)x, rows, cols, tiles_c, s, out_row, out_t, margin, mu_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cast(const void* x, int64_t rows, int64_t cols, int fmt, const fp8_scale_t* s,
                       uint8_t* out_row, uint8_t* out_t, hipStream_t st) {
  if (rows == 0 || cols == 0 || (!out_row && !out_t)) return hipSuccess;
  return launch_cast_t<false>(x, rows, cols, fmt, const_cast<fp8_scale_t*>(s), out_row, out_t, 0, 0, st);
}

hipError_t launch_quantize(const void* x, int64_t rows, int64_t cols, int fmt, int margin, int mu_log2,
                           fp8_scale_t* s, uint8_t* out_row, uint8_t* out_t, hipStream_t st) {
  hipError_t e = launch_amax_gen(x, rows * cols, s, st);
  if (e != hipSuccess) return e;
  if (rows == 0 || cols == 0 || (!out_row && !out_t)) {
    // nothing to cast: one block with no rows still publishes the record
    return launch_cast_t<true>(x, 0, 0, fmt, s, nullptr, nullptr, margin, mu_log2, st);
  }
  return launch_cast_t<true>(x, rows, cols, fmt, s, out_row, out_t, margin, mu_log2, st);
}

hipError_t launch_quantize_batch(const QuantDesc* d, int count, hipStream_t st) {
  if (count < 1 || count > kQuantBatchMax) return hipErrorInvalidValue;
  hipError_t e = launch_amax_batch(d, count, st);
  if (e != hipSuccess) return e;
  CastBatch b{};
  b.count = count;
  int blocks = 0;
  for (int i = 0; i < count; ++i) {
    CastEntry& c = b.e[i];
    const bool empty = d[i].rows == 0 || d[i].cols == 0 || (!d[i].out_row && !d[i].out_t);
    c.x = (const uint16_t*)d[i].x;
    c.rows = empty ? 0 : d[i].rows;
    c.cols = empty ? 0 : d[i].cols;
    c.tiles_c = empty ? 1 : (d[i].cols + kTile - 1) / kTile;
    c.s = d[i].s;
    c.out_row = empty ? nullptr : d[i].out_row;
    c.out_t = empty ? nullptr : d[i].out_t;
    c.fmt = d[i].fmt;
    c.margin = d[i].margin;
    c.mu_log2 = d[i].mu_log2;
    c.first_block = blocks;
    // an empty tensor: one block that reads nothing and publishes the record
    blocks += empty ? 1 : (int)(((d[i].rows + kTile - 1) / kTile) * c.tiles_c);
  }
  hipLaunchKernelGGL(cast_batch_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_quantize_spec(const void* x, int64_t rows, int64_t cols, int fmt, int margin, int mu_log2,
                                fp8_scale_t* s, uint8_t* out_row, hipStream_t st) {
  int64_t tiles_r = (rows + kTile - 1) / kTile, tiles_c = (cols + kTile - 1) / kTile;
  if (tiles_r * tiles_c == 0) tiles_r = tiles_c = 1;  // empty: one block that reads nothing
  const int64_t ntiles = tiles_r * tiles_c;
  // at most kSpecBlocks blocks of kSpecGroups tile groups, looping over
  // tiles: one merge per block. The check runs one block per tile up to
  // the same cap (it only recasts when the guess was wrong).
  const int64_t sblocks = (ntiles + kSpecGroups - 1) / kSpecGroups;
  const dim3 sgrid((unsigned)(sblocks < kSpecBlocks ? sblocks : kSpecBlocks));
  const dim3 grid((unsigned)(ntiles < kSpecBlocks ? ntiles : kSpecBlocks));
  const uint16_t* xp = (const uint16_t*)x;
  if (fmt == FP8_E4M3) {
    hipLaunchKernelGGL((quantize_spec_kernel<FP8_E4M3>), sgrid, dim3(kThreads * kSpecGroups), 0, st, xp, rows,
                       cols, tiles_c, ntiles, s, out_row);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((quantize_check_kernel<FP8_E4M3>), grid, dim3(kThreads), 0, st, xp, rows, cols, tiles_c,
                       ntiles, s, out_row, margin, mu_log2);
  } else {
    hipLaunchKernelGGL((quantize_spec_kernel<FP8_E5M2>), sgrid, dim3(kThreads * kSpecGroups), 0, st, xp, rows,
                       cols, tiles_c, ntiles, s, out_row);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((quantize_check_kernel<FP8_E5M2>), grid, dim3(kThreads), 0, st, xp, rows, cols, tiles_c,
                       ntiles, s, out_row, margin, mu_log2);
  }
  return hipGetLastError();
}

hipError_t launch_wgrad_cast(const void* dw, int64_t rows, int64_t cols, fp8_scale_t* s, uint8_t* out_row,
                             uint8_t* out_t, int margin, int mu_log2, hipStream_t st) {
  return launch_cast_t<true, true>(dw, rows, cols, FP8_E5M2, s, out_row, out_t, margin, mu_log2, st);
}

}  // namespace fp8lin
