// a4-a6 FP8 GEMM, NT form, on CDNA4 FP8/BF8 MFMA with FP32 accumulation and
// a dequantising bf16 epilogue:
//   C[i, j] = bf16_rne( 2^-(bias_a + bias_b) * sum_r A[i, r] * B[j, r] )
// [Perez et al. review, "Proposed method", bullet 3: the matmul runs on the
// scaled FP8 operands and the scaling is undone after it; bullet 4: E4 for
// weights/activations, E5 for gradients, so the backward GEMMs mix formats].
//
// Design for gfx950:
//  * v_mfma_f32_32x32x64_f8f6f4: one instruction per 32 x 32 x 64 block, the
//    A and B formats chosen independently (E4M3 or E5M2), so the mixed
//    E5M2 x E4M3 backward GEMMs need no conversion. Each lane feeds 32
//    consecutive k-bytes of one row; A and B use the same k assignment, so
//    every product pairs equal k.
//  * 256 x 256 output tile per 256-thread block (4 waves, 2 x 2), each wave
//    128 x 128 = 4 x 4 MFMA blocks (256 FP32 accumulators per lane, held in
//    the accumulation registers). k advances 128 bytes per stage.
//  * Operands staged through LDS, double buffered (2 x 64 KB): the next
//    stage's global loads (16-byte, whole 128-byte lines) are in flight while
//    the current stage is multiplied, then written to the other buffer; one
//    barrier per stage. 16-byte chunks of each 128-byte LDS row are
//    XOR-swizzled so fragment reads of 8 (or 16) consecutive rows hit
//    distinct banks.
//  * The MFMA is fed B as its first operand and A as its second, so it
//    produces C^T blocks: each lane then holds 4 runs of 4 consecutive
//    output columns of one row, stored as 8-byte pieces.
//  * Tiles are numbered so that each XCD (workgroups are dealt round-robin
//    over the 8 XCDs) works on one contiguous, row-grouped region of C and
//    its operand panels stay in that XCD's L2.
//  * Rows past M or N read a clamped (valid) row and are never stored; k
//    past R is zero-filled, so any M, N, R that are multiples of 16 work.
#include "fp8lin_internal.h"

namespace fp8lin {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 128;  // tile rows, tile cols, k-bytes per stage
constexpr int kThreads = 256;
constexpr int kGroupM = 8;                      // tile rows per raster group
constexpr int kStageBytes = (kBM + kBN) * kBK;  // 64 KB

__device__ inline int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ inline uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int FA, int FB>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, const fp8_scale_t* __restrict__ sa,
    const fp8_scale_t* __restrict__ sb, int64_t M, int64_t N, int64_t R, uint16_t* __restrict__ C,
    int tiles_m, int tiles_n) {
  __shared__ uint4 smem[2 * kStageBytes / 16];

  // ---- tile selection: XCD-contiguous ranges, grouped raster inside ----
  const int nblocks = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if ((nblocks & 7) == 0) pid = (pid & 7) * (nblocks >> 3) + (pid >> 3);
  const int per_group = kGroupM * tiles_n;
  const int group = pid / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = pid - group * per_group;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;

  // ---- global -> register loads: thread t owns chunk (t & 7) of rows (t >> 3) + 32 i ----
  const int lrow = t >> 3, lch = t & 7;
  const uint8_t* pa[8];
  const uint8_t* pb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t ra = min(m0 + lrow + 32 * i, M - 1);
    const int64_t rb = min(n0 + lrow + 32 * i, N - 1);
    pa[i] = A + ra * R + 16 * lch;
    pb[i] = B + rb * R + 16 * lch;
  }
  const int wsw = (lrow & 7) ^ ((lrow >> 3) & 1);  // swz() of every row this thread writes
  const int wr_off = lrow * kBK + ((lch ^ wsw) << 4);

  uint4 ra[8], rb[8];
  auto load_stage = [&](int64_t k0) {
    const bool kv = k0 + 16 * lch < R;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ra[i] = kv ? *(const uint4*)(pa[i] + k0) : make_uint4(0, 0, 0, 0);
      rb[i] = kv ? *(const uint4*)(pb[i] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* base = (uint8_t*)smem + buf * kStageBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *(uint4*)(base + wr_off + i * 32 * kBK) = ra[i];
      *(uint4*)(base + kBM * kBK + wr_off + i * 32 * kBK) = rb[i];
    }
  };

  // ---- fragment reads: lane -> row (lane & 31), k-bytes 32*(lane >> 5) of each 64-byte half ----
  const int frow = lane & 31, g = lane >> 5;
  auto read_frag = [&](const uint8_t* base, int row, int s) -> v8i {
    const int c0 = 4 * s + 2 * g;
    const int sw = swz(row);
    const uint4 lo = *(const uint4*)(base + row * kBK + ((c0 ^ sw) << 4));
    const uint4 hi = *(const uint4*)(base + row * kBK + (((c0 + 1) ^ sw) << 4));
    v8i v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
  };

  v16f acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

  const int64_t nk = (R + kBK - 1) / kBK;
  if (nk > 0) {
    load_stage(0);
    store_stage(0);
    __syncthreads();
  }
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    if (kt + 1 < nk) load_stage((kt + 1) * kBK);
    const uint8_t* as = (const uint8_t*)smem + cur * kStageBytes;
    const uint8_t* bs = as + kBM * kBK;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v8i af[4], bf[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) af[mi] = read_frag(as, 128 * wm + 32 * mi + frow, s);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) bf[ni] = read_frag(bs, 128 * wn + 32 * ni + frow, s);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[ni], af[mi], acc[mi][ni],
                                                                         FB, FA, 0, 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: 2^-(ba+bb) (exact power-of-two scaling), bf16 RNE, 8-byte stores ----
  const int shift = -(sa->bias + sb->bias);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int64_t row = m0 + 128 * wm + 32 * mi + frow;
    if (row >= M) continue;
    uint16_t* crow = C + row * N;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n0 + 128 * wn + 32 * ni + 8 * q + 4 * g;
        if (col < N) {
          const float f0 = ldexpf(acc[mi][ni][4 * q + 0], shift);
          const float f1 = ldexpf(acc[mi][ni][4 * q + 1], shift);
          const float f2 = ldexpf(acc[mi][ni][4 * q + 2], shift);
          const float f3 = ldexpf(acc[mi][ni][4 * q + 3], shift);
          const uint32_t p0 = f32_to_bf16_rne(f0) | (f32_to_bf16_rne(f1) << 16);
          const uint32_t p1 = f32_to_bf16_rne(f2) | (f32_to_bf16_rne(f3) << 16);
          *(uint2*)(crow + col) = make_uint2(p0, p1);
        }
      }
    }
  }
}

template <int FA, int FB>
hipError_t launch_typed(const uint8_t* A, const fp8_scale_t* sa, const uint8_t* B, const fp8_scale_t* sb,
                        int64_t M, int64_t N, int64_t R, void* C, hipStream_t st) {
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
  hipLaunchKernelGGL((gemm_nt_kernel<FA, FB>), dim3(tiles_m * tiles_n), dim3(kThreads), 0, st, A, B,
                     sa, sb, M, N, R, (uint16_t*)C, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t* A, int fa, const fp8_scale_t* sa, const uint8_t* B, int fb,
                       const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R, void* C,
                       hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (fa == FP8_E4M3 && fb == FP8_E4M3) return launch_typed<0, 0>(A, sa, B, sb, M, N, R, C, st);
  if (fa == FP8_E5M2 && fb == FP8_E4M3) return launch_typed<1, 0>(A, sa, B, sb, M, N, R, C, st);
  if (fa == FP8_E4M3 && fb == FP8_E5M2) return launch_typed<0, 1>(A, sa, B, sb, M, N, R, C, st);
  return launch_typed<1, 1>(A, sa, B, sb, M, N, R, C, st);
}

}  // namespace fp8lin
