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
//    the accumulation registers).
//  * Operands stream through a 4-slot LDS ring of k = 64-byte stages
//    (32 KB each: 256 rows of A and of B). Global memory is copied straight
//    into LDS by 16-byte direct-to-LDS loads (no register staging), issued
//    four stages ahead of use. With one wave per SIMD nothing else hides
//    the non-MFMA work, so each stage is software-pipelined: the first half
//    of its 16 MFMAs runs on fragments already in registers; then the next
//    stage's loads are awaited (in-order vmcnt), one barrier frees the
//    current slot, the loads of stage+4 are issued into it and the next
//    stage's fragments are read, all under the second half of the MFMAs.
//  * A direct-to-LDS load writes lane l's 16 bytes at slot l of a 1 KB LDS
//    block (16 rows x 64 bytes), so the bank swizzle is applied on the
//    source side: the lane for LDS chunk p of row r fetches global chunk
//    p ^ swz(r). Fragment reads then hit distinct banks.
//  * The MFMA is fed B as its first operand and A as its second, so it
//    produces C^T blocks: each lane then holds 4 runs of 4 consecutive
//    output columns of one row. The epilogue scales by 2^-(ba+bb), packs
//    pairs to bf16 with the hardware round-to-nearest-even converter,
//    stages the tile in LDS and writes C in whole rows (scattered 8-byte
//    stores would leave partial cache lines and multiply HBM writes).
//  * Tiles are numbered so that each XCD (workgroups are dealt round-robin
//    over the 8 XCDs) works on one contiguous, row-grouped region of C and
//    its operand panels stay in that XCD's L2.
//  * Rows past M or N read a clamped (valid) row and are never stored; k
//    past R is zero-filled in LDS, so any M, N, R that are multiples of 16
//    work.
#include <type_traits>

#include "fp8lin_internal.h"

namespace fp8lin {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 256, kBN = 256, kBK = 64;   // tile rows, tile cols, k-bytes per stage
constexpr int kThreads = 256;
constexpr int kGroupM = 8;                       // tile rows per raster group
constexpr int kStages = 4;                       // LDS ring slots (all four hold stages in flight)
constexpr int kStageBytes = (kBM + kBN) * kBK;   // 32 KB
constexpr int kLoadsPerStage = 8;                // direct-to-LDS loads per thread per stage

#define LDS_AS __attribute__((address_space(3)))
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef LDS_AS uint8_t lds_u8;
typedef LDS_AS u32x4 lds_u32x4;
typedef LDS_AS u32x2 lds_u32x2;

// 16-byte chunk swizzle of a 64-byte LDS row (four rows share one 256-byte
// bank line). A fragment read has each lane take chunk 2g or 2g+1 of row
// (lane & 31), g = lane >> 5. With swz = (row >> 2) & 3, the 16 rows of a
// 16-lane group at one chunk land on 16 distinct 16-byte bank groups, and
// so do 8 rows x both halves (chunks c, c+2) when lanes l and l+32 are
// served together: swz(r) ^ swz(r+4) always has bit 0 set.
__device__ inline int swz(int row) { return (row >> 2) & 3; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt 7 and lgkmcnt 15 = no wait)
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ inline void wait_loads_after(int n_after_full) {
  // stages issued after the one to be consumed, each kLoadsPerStage loads
  if (n_after_full >= 3) wait_vmcnt<3 * kLoadsPerStage>();
  else if (n_after_full == 2) wait_vmcnt<2 * kLoadsPerStage>();
  else if (n_after_full == 1) wait_vmcnt<kLoadsPerStage>();
  else wait_vmcnt<0>();
}

__device__ inline void block_sync_lds() {
  // all LDS writes of this wave done, then the workgroup barrier; the empty
  // asm keeps the compiler from moving memory accesses across it
  __builtin_amdgcn_s_waitcnt((63 & 15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int FA, int FB>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, const fp8_scale_t* __restrict__ sa,
    const fp8_scale_t* __restrict__ sb, int M, int N, int R, uint16_t* __restrict__ C, int tiles_m,
    int tiles_n) {
  // The ring's four slots are four separate LDS objects, always addressed
  // with a compile-time slot index, so the compiler can tell the slot being
  // read from the slots with loads in flight and does not wait for those.
  __shared__ uint4 slot0[kStageBytes / 16], slot1[kStageBytes / 16], slot2[kStageBytes / 16],
      slot3[kStageBytes / 16];
  auto slot = [&](auto J_) -> lds_u8* {
    constexpr int J = decltype(J_)::value % kStages;
    if constexpr (J == 0) return (lds_u8*)slot0;
    else if constexpr (J == 1) return (lds_u8*)slot1;
    else if constexpr (J == 2) return (lds_u8*)slot2;
    else return (lds_u8*)slot3;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

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
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, scalar
  const int wm = w >> 1, wn = w & 1;

  // ---- direct-to-LDS loads: wave w fills 1 KB blocks 4w..4w+3 of the A and
  // B halves of a stage; lane l of block b writes row 16b + l/4, LDS chunk
  // l%4. Operands are below 4 GiB, so per-lane offsets are 32-bit.
  uint32_t offa[4], offb[4];
  int kc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * (4 * w + i) + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    kc[i] = 16 * c;
    offa[i] = (uint32_t)min(m0 + row, M - 1) * (uint32_t)R + kc[i];
    offb[i] = (uint32_t)min(n0 + row, N - 1) * (uint32_t)R + kc[i];
  }
  const int nk = (R + kBK - 1) / kBK;      // k-stages
  const int nfull = R / kBK;               // full k-stages (all but a partial last one)

  // loads of one full stage: 4 of A, 4 of B per thread
  auto issue_full = [&](lds_u8* sl, int stage) {
    const uint8_t* a0 = A + stage * kBK;  // wave-uniform bases; per-lane offsets
    const uint8_t* b0 = B + stage * kBK;
    lds_u8* sbase = sl + (4 * w) * 1024;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_global_load_lds((const void*)(a0 + offa[i]), (LDS_AS void*)(sbase + i * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(b0 + offb[i]), (LDS_AS void*)(sbase + kBM * kBK + i * 1024),
                                       16, 0, 0);
    }
  };
  // any stage, including a partial last one (k past R zero-filled)
  auto issue_any = [&](lds_u8* sl, int stage) {
    if (stage < nfull) {
      issue_full(sl, stage);
      return;
    }
    const int k0 = stage * kBK;
    const uint8_t* a0 = A + k0;
    const uint8_t* b0 = B + k0;
    lds_u8* sbase = sl + (4 * w) * 1024;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lds_u8* da = sbase + i * 1024;
      lds_u8* db = sbase + kBM * kBK + i * 1024;
      if (k0 + kc[i] < R) {
        __builtin_amdgcn_global_load_lds((const void*)(a0 + offa[i]), (LDS_AS void*)da, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(b0 + offb[i]), (LDS_AS void*)db, 16, 0, 0);
      } else {
        *(lds_u32x4*)(da + 16 * lane) = (u32x4){0, 0, 0, 0};
        *(lds_u32x4*)(db + 16 * lane) = (u32x4){0, 0, 0, 0};
      }
    }
  };

  // ---- fragment reads: lane -> row (lane & 31), logical chunks 2g, 2g+1 ----
  // swz() of every fragment row equals swz(lane & 31) (fragment rows start at
  // multiples of 32), so two per-lane offsets plus compile-time immediates
  // address every fragment of every slot.
  const int frow = lane & 31, g = lane >> 5;
  const int fsw = swz(frow);
  const int off_lo = frow * kBK + (((2 * g) ^ fsw) << 4);
  const int off_hi = frow * kBK + (((2 * g + 1) ^ fsw) << 4);
  const int a_row0 = 128 * wm * kBK, b_row0 = kBM * kBK + 128 * wn * kBK;  // wave-uniform
  struct Frags {
    v8i a[4], b[4];
  };
  auto read_frag = [&](const lds_u8* p) -> v8i {
    const u32x4 lo = *(const lds_u32x4*)(p + off_lo);
    const u32x4 hi = *(const lds_u32x4*)(p + off_hi);
    v8i v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
  };
  auto read_stage = [&](const lds_u8* sl, Frags& f) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) f.b[ni] = read_frag(sl + b_row0 + 32 * ni * kBK);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) f.a[mi] = read_frag(sl + a_row0 + 32 * mi * kBK);
  };

  v16f acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

  auto mfma_rows = [&](const Frags& f, int mlo) {
#pragma unroll
    for (int mi = mlo; mi < mlo + 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[ni], f.a[mi], acc[mi][ni], FB, FA,
                                                                       0, 0, 0, 0);
  };
  // wait until stage `st` has landed when stages up to `newest` are issued;
  // the count of younger loads is exact only if they are all full stages
  auto wait_for_stage = [&](int st, int newest) {
    const bool full = newest < nfull;
    wait_loads_after(full ? newest - st : 0);
  };

  // Software pipeline over k-stages. On entry to stage kt its fragments are
  // in registers (fr[kt & 1]). The first half of its MFMAs runs, then:
  // stage kt+1's loads are awaited, one barrier (every wave has finished
  // reading slot kt), the loads of stage kt+4 go into that slot, and stage
  // kt+1's fragments are read into the other register set while the second
  // half of stage kt's MFMAs runs.
  Frags fr[2];
  if (nk > 0) issue_any(slot(S0{}), 0);
  if (nk > 1) issue_any(slot(S1{}), 1);
  if (nk > 2) issue_any(slot(S2{}), 2);
  if (nk > 3) issue_any(slot(S3{}), 3);
  if (nk > 0) {
    wait_for_stage(0, min(3, nk - 1));
    block_sync_lds();
    read_stage(slot(S0{}), fr[0]);
  }
  // steady state: every stage touched is full, stage kt+4 exists. Hard
  // scheduling fences keep the order: first-half MFMAs | wait + barrier |
  // loads of stage kt+4 and fragment reads of stage kt+1 interleaved with
  // the second-half MFMAs (two reads, one load, one MFMA per slot).
  auto step_main = [&](auto J_, int kt) {
    constexpr int J = decltype(J_)::value;
    Frags& cur = fr[J & 1];
    Frags& nxt = fr[(J + 1) & 1];
    mfma_rows(cur, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<2 * kLoadsPerStage>();  // stage kt+1 landed (kt+2, kt+3 may be in flight)
    block_sync_lds();
    __builtin_amdgcn_sched_barrier(0);
    issue_full(slot(J_), kt + 4);
    read_stage(slot(std::integral_constant<int, J + 1>{}), nxt);
    mfma_rows(cur, 2);
    // reads first in each slot, so the last fragment reads are in flight
    // before the last MFMA of the stage is issued
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read (direct-to-LDS)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // general step (tail): bounds on every stage
  auto step_any = [&](auto J_, int kt) {
    constexpr int J = decltype(J_)::value;
    Frags& cur = fr[J & 1];
    Frags& nxt = fr[(J + 1) & 1];
    mfma_rows(cur, 0);
    if (kt + 1 < nk) {
      wait_for_stage(kt + 1, min(kt + 3, nk - 1));
      block_sync_lds();
      if (kt + 4 < nk) issue_any(slot(J_), kt + 4);
      read_stage(slot(std::integral_constant<int, J + 1>{}), nxt);
    }
    mfma_rows(cur, 2);
  };
  const int main_steps = nfull >= 4 ? ((nfull - 4) & ~(kStages - 1)) : 0;  // multiple of 4
  int kt = 0;
  for (; kt < main_steps; kt += kStages) {
    step_main(S0{}, kt);
    step_main(S1{}, kt + 1);
    step_main(S2{}, kt + 2);
    step_main(S3{}, kt + 3);
  }
  for (; kt < nk; kt += kStages) {
    step_any(S0{}, kt);
    if (kt + 1 < nk) step_any(S1{}, kt + 1);
    if (kt + 2 < nk) step_any(S2{}, kt + 2);
    if (kt + 3 < nk) step_any(S3{}, kt + 3);
  }
  wait_vmcnt<0>();
  block_sync_lds();

  // ---- epilogue: 2^-(ba+bb) (exact power-of-two scaling), bf16 RNE, then
  // the 256 x 256 bf16 tile (128 KB: 64 rows of 512 bytes per slot) is
  // staged row-major in LDS so the block writes C in whole 512-byte rows of
  // 16-byte stores. 16-byte chunks of each LDS row are XOR-swizzled by
  // (row & 31).
  const int shift = -(sa->bias + sb->bias);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int row = 128 * wm + 32 * mi + frow;
    lds_u8* crow = (mi < 2 ? (wm ? slot(S2{}) : slot(S0{})) : (wm ? slot(S3{}) : slot(S1{}))) +
                   (row & 63) * 512;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x2 lo = {ldexpf(acc[mi][ni][4 * q + 0], shift), ldexpf(acc[mi][ni][4 * q + 1], shift)};
        f32x2 hi = {ldexpf(acc[mi][ni][4 * q + 2], shift), ldexpf(acc[mi][ni][4 * q + 3], shift)};
        const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
        const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
        const int chunk = 16 * wn + 4 * ni + q;
        *(lds_u32x2*)(crow + ((chunk ^ (row & 31)) << 4) + 8 * g) = (u32x2){p0, p1};
      }
    }
  }
  block_sync_lds();
  auto drain = [&](const lds_u8* src, int j) {
#pragma unroll 4
    for (int k = 0; k < 8; ++k) {
      const int q = t + kThreads * k;        // 2048 chunks of 16 bytes per slot
      const int lrow = q >> 5, c = q & 31;   // 64 rows x 32 chunks
      const int row = 64 * j + lrow;
      const u32x4 v = *(const lds_u32x4*)(src + lrow * 512 + ((c ^ (row & 31)) << 4));
      const int grow = m0 + row, gcol = n0 + 8 * c;
      if (grow < M && gcol < N) *(u32x4*)(C + (int64_t)grow * N + gcol) = v;
    }
  };
  drain(slot(S0{}), 0);
  drain(slot(S1{}), 1);
  drain(slot(S2{}), 2);
  drain(slot(S3{}), 3);
}

template <int FA, int FB>
hipError_t launch_typed(const uint8_t* A, const fp8_scale_t* sa, const uint8_t* B, const fp8_scale_t* sb,
                        int64_t M, int64_t N, int64_t R, void* C, hipStream_t st) {
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
  hipLaunchKernelGGL((gemm_nt_kernel<FA, FB>), dim3(tiles_m * tiles_n), dim3(kThreads), 0, st, A, B,
                     sa, sb, (int)M, (int)N, (int)R, (uint16_t*)C, tiles_m, tiles_n);
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
