// a4-a6 FP8 GEMM on CDNA4 FP8/BF8 MFMA with FP32 accumulation and a
// dequantising bf16 epilogue:
//   C[i, j] = bf16_rne( 2^-(bias_a + bias_b) * sum_r A(i, r) * B(j, r) )
// with each operand stored either with one row per output index and the
// reduction contiguous (A [M, R], B [N, R]) or reduction-major (A [R, M],
// B [R, N]: a row-major FP8 copy read transposed), so the forward, dgrad
// and wgrad GEMMs all read the same row-major copies of X, W and dY.
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
//  * Operands stream through LDS in stages of k = 128 bytes (256 rows of A
//    and of B, 32 KB each), held in two slots for A and three for B (160 KB),
//    so B, the operand streamed from HBM, is loaded a stage and a half
//    ahead and A one. 128 bytes is one cache line per row: a 16-byte-per-lane load then
//    covers 8 whole lines, which the load path handles markedly faster than
//    16 half lines. Global memory is copied straight into LDS by buffer
//    loads with the LDS-write form (no register staging).
//  * Each stage is two MFMA steps of k = 64 (16 MFMAs per wave each). With
//    one wave per SIMD nothing else hides the non-MFMA work, so the steps
//    are software-pipelined: fragments of the next step are read from LDS
//    into a second register set under the current step's MFMAs. One
//    barrier per stage: at the second step of stage s, stage s+1 is awaited,
//    and the loads of A of stage s+2 and B of stage s+3 go into the slots of
//    stage s, whose fragments every wave has read by then.
//  * A load writes lane l's 16 bytes at slot l of a 1 KB LDS block (8 rows
//    x 128 bytes), so the bank swizzle is applied on the source side: the
//    lane for LDS chunk p of row r fetches global chunk p ^ swz(r).
//    Fragment reads then hit distinct banks.
//  * The MFMA is fed B as its first operand and A as its second, so it
//    produces C^T blocks: each lane then holds 4 runs of 4 consecutive
//    output columns of one row. The epilogue scales by 2^-(ba+bb), packs
//    pairs to bf16 with the hardware round-to-nearest-even converter, and
//    each wave stages its block in LDS a quarter at a time and writes C in
//    whole 256-byte row pieces (scattered 8-byte stores would leave partial
//    cache lines and multiply HBM writes); a quarter's stores drain while
//    the next is converted. The stores are nontemporal: C is written once
//    and read by a later kernel, and streaming it out during the GEMM keeps
//    the write-back of its dirty lines out of the kernels that follow.
//  * Tiles are numbered so that each XCD (workgroups are dealt round-robin
//    over the 8 XCDs) works on one contiguous, row-grouped region of C and
//    its operand panels stay in that XCD's L2.
//  * Reduction-major operands are staged as [k][output] and turned into
//    the same fragments by transposing LDS reads (ds_read_b64_tr_b8), so
//    the MFMAs see identical operands in either layout.
//  * Rows past M or N read a clamped (valid) row and are never stored; k
//    past R is zero-filled in LDS, so any M, N, R that are multiples of 16
//    work.
//  * The per-tile body is one force-inlined function, so a launch can run
//    tiles of two GEMMs (gemm_pair_kernel: a linear's dgrad then its
//    wgrad, whose tiles fill the dgrad's last wave) or split the tiles of a
//    last wave at most half full into two reduction halves
//    (gemm_tailsplit_kernel: FP32 partials in a caller workspace, added by
//    gemm_tail_fixup_kernel), with the per-tile arithmetic unchanged.
//  * Two bodies of the same tile. The chip runs these GEMMs at its power
//    limit, and v_mfma_f32_16x16x128_f8f6f4 spends less energy per FLOP
//    than the 32 x 32 x 64 instruction (a register-only probe over all CUs
//    sustains ~10 % more FLOP/s with random FP8 data), which shows as a
//    higher clock. gemm_tile16 uses it wherever A has one row per output
//    index (forward, dgrad, the inference forward): a stage is 64 MFMAs per
//    wave, each consuming the whole k = 128 of a 16 x 16 block, with the A
//    and B fragments refilled in place or double-buffered in registers
//    under the MFMAs. With a reduction-major A (wgrad) its fragment
//    registers and the transposing reads' addresses no longer fit beside
//    the accumulators, so gemm_tile (32 x 32 x 64) serves those layouts.
//    Each layout always takes the same body, so a result never depends on
//    the launch (single, pair, tail split); the two bodies round FP32
//    partial sums at different k boundaries, so a row-layout and a
//    reduction-major A can differ in the last bf16 bit of rare elements.
#include <mutex>
#include <type_traits>

#include "fp8lin_internal.h"

namespace fp8lin {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 256, kBN = 256;
constexpr int kBK = 128;                         // k-bytes per stage (one cache line per row)
constexpr int kThreads = 256;
constexpr int kGroupM = 8;                       // tile rows per raster group
constexpr int kOpBytes = kBM * kBK;              // 32 KB: the A (or B) part of a stage
constexpr int kRsrcWord3 = 0x00020000;           // buffer resource word 3 for raw byte loads (gfx9 family)

#define LDS_AS __attribute__((address_space(3)))
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef LDS_AS uint8_t lds_u8;
typedef LDS_AS u32x4 lds_u32x4;
typedef LDS_AS u32x2 lds_u32x2;
typedef LDS_AS v2i lds_v2i;

// 16-byte chunk swizzle of a 128-byte LDS row (two rows share one 256-byte
// bank line). A fragment read has each lane take one chunk of row
// (lane & 31); with swz = (row >> 1) & 7, the 16 rows of a 16-lane group at
// one logical chunk land on 16 distinct 16-byte bank groups (row & 1 picks
// the half of the bank line, the swizzled chunk the group within it).
__device__ inline int swz(int row) { return (row >> 1) & 7; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt 7 and lgkmcnt 15 = no wait)
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// calls f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>) in order
template <int N, int I = 0, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

__device__ inline void block_sync_lds() {
  // all LDS writes of this wave done, then the workgroup barrier; the empty
  // asm keeps the compiler from moving memory accesses across it
  __builtin_amdgcn_s_waitcnt((63 & 15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One GEMM problem: operands, records, sizes and the tile grid.
struct GemmParams {
  const uint8_t* A;
  const uint8_t* B;
  const fp8_scale_t* sa;
  const fp8_scale_t* sb;
  uint16_t* C;
  int M, N, R, tiles_m, tiles_n;
};

// Stage buffers: two slots for A's part of a stage and three for B's
// (32 KB each, 160 KB in all, the whole LDS of a CU), so B's loads are
// issued half a stage earlier than A's. B is the operand streamed from HBM
// on the layer shapes (the weights in the forward and dgrad GEMMs, the
// gradient in the wgrad), whose latency one stage of lead did not cover.
// They are separate LDS objects, always addressed with a compile-time
// index, so the compiler can tell a slot being read from one with loads in
// flight and does not wait for those. B2 also stages the epilogue's C
// quarters (8 KB per wave), and A0, A1, B0, B1 the tail fixup's C tile.
// Declared once for the file, so a kernel that runs tiles of two GEMM
// variants still holds 160 KB.
__shared__ uint4 g_a0[kOpBytes / 16];
__shared__ uint4 g_a1[kOpBytes / 16];
__shared__ uint4 g_b0[kOpBytes / 16];
__shared__ uint4 g_b1[kOpBytes / 16];
__shared__ uint4 g_b2[kOpBytes / 16];

// A slot of stage s (s % 2) and B slot (s % 3), for compile-time s
template <int S>
__device__ inline lds_u8* a_slot() {
  if constexpr (S % 2 == 0) return (lds_u8*)g_a0;
  else return (lds_u8*)g_a1;
}
template <int S>
__device__ inline lds_u8* b_slot() {
  if constexpr (S % 3 == 0) return (lds_u8*)g_b0;
  else if constexpr (S % 3 == 1) return (lds_u8*)g_b1;
  else return (lds_u8*)g_b2;
}
// 32 KB region j (0..3) of the tail fixup's C staging: A0, A1, B0, B1
__device__ inline lds_u8* c_region(int j) {
  return j == 0 ? (lds_u8*)g_a0 : j == 1 ? (lds_u8*)g_a1 : j == 2 ? (lds_u8*)g_b0 : (lds_u8*)g_b1;
}

// AMAX: the epilogue also takes max |C| over the bf16 values it writes and
// merges (tag << 16) | max into s_out->gen_max (one atomic per block, as the
// amax pass of fp8_quantize does; tag = s_out->epoch + 1), so a following
// derive-cast of C needs no amax pass; block 0 also clears
// s_out->sat_count for that cast.
// TA / TB: operand layout. false: one row per output index with the R
// reduction bytes contiguous (A [M, R], B [N, R]); true: reduction-major
// (A [R, M], B [R, N]), staged in LDS as [k][output] and turned into MFMA
// fragments by transposing LDS reads.
// Tile order: workgroups are dealt round-robin to the 8 XCDs, so index
// pid runs on XCD pid % 8; each XCD gets one contiguous range of tiles
// (when the count is a multiple of 8), rastered in groups of kGroupM tile
// rows so that an XCD's concurrent tiles share operand panels in its L2.
__device__ inline void tile_origin(int pid, int tiles_m, int tiles_n, int& m0, int& n0) {
  const int nblocks = tiles_m * tiles_n;
  if ((nblocks & 7) == 0) pid = (pid & 7) * (nblocks >> 3) + (pid >> 3);
  const int per_group = kGroupM * tiles_n;
  const int group = pid / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = pid - group * per_group;
  m0 = (first_m + in_group % gsize) * kBM;
  n0 = (in_group / gsize) * kBN;
}

// tile: index of the output tile within the problem's tile grid.
// HALF: the block takes reduction half `half` of the tile (stages
// [half * nk / 2, (half + 1) * nk / 2), R a multiple of 256) and, instead
// of the epilogue, stores its unscaled FP32 sums to `part` (65536 floats,
// in register order: float4 r4 = (mi * 4 + ni) * 4 + q of thread t at
// float offset 1024 r4 + 4 t); gemm_tail_fixup_kernel<false> adds the two halves.
template <int FA, int FB, bool AMAX, bool TA, bool TB, bool HALF = false>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, int tile, fp8_scale_t* s_out, int half = 0,
                                          float* part = nullptr) {
  const uint8_t* __restrict__ A = p.A;
  const uint8_t* __restrict__ B = p.B;
  const fp8_scale_t* __restrict__ sa = p.sa;
  const fp8_scale_t* __restrict__ sb = p.sb;
  uint16_t* __restrict__ C = p.C;
  const int M = p.M, N = p.N, R = p.R, tiles_m = p.tiles_m, tiles_n = p.tiles_n;

  // ---- tile selection: XCD-contiguous ranges, grouped raster inside ----
  int m0, n0;
  tile_origin(tile, tiles_m, tiles_n, m0, n0);

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, scalar
  const int wm = w >> 1, wn = w & 1;

  // ---- loads: wave w fills 1 KB blocks 8w..8w+7 of the A and B parts of a
  // stage (a part is 32 KB). Row-layout operand: lane l of block b writes
  // row 8b + l/8 (an output index), LDS chunk l%8, which holds global chunk
  // (l%8) ^ swz(row) of that row's 128 k-bytes; rows past M / N read the
  // last valid row. Reduction-major operand: lane l of block b writes k-row
  // 4b + l/16, LDS chunk l%16 of that row's 256 output bytes, which holds
  // global chunk (l%16) ^ (krow & 7); chunks past M / N read the last valid
  // chunk, so the tile only ever holds real operand values. Operands are
  // below 4 GiB, so per-lane offsets are 32-bit; the stage offset is a
  // scalar (stage * 128 for rows, stage * 128 * M or N for reduction-major).
  // op_offset: product part p (laundered below) and added part c of lane's
  // offset for load i.
  auto op_offset = [&](auto T_, int i, int o0, int O, uint32_t& p, uint32_t& c) {
    if constexpr (!decltype(T_)::value) {
      const int row = 8 * (8 * w + i) + (lane >> 3);
      p = (uint32_t)min(o0 + row, O - 1) * (uint32_t)R;
      c = 16 * ((lane & 7) ^ swz(row));
    } else {
      const int krow = 4 * (8 * w + i) + (lane >> 4);
      p = (uint32_t)krow * (uint32_t)O;
      c = (uint32_t)min(o0 + 16 * ((lane & 15) ^ (krow & 7)), O - 16);
    }
  };
  using TAc = std::integral_constant<bool, TA>;
  using TBc = std::integral_constant<bool, TB>;
  uint32_t offa[8], offb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // 32-bit products, passed through an empty asm: fused into a 64-bit
    // multiply-add, each offset would occupy a register pair
    uint32_t pa, ca, pb, cb;
    op_offset(TAc{}, i, m0, M, pa, ca);
    op_offset(TBc{}, i, n0, N, pb, cb);
    asm volatile("" : "+v"(pa), "+v"(pb));
    offa[i] = pa + ca;
    offb[i] = pb + cb;
  }
  // stages of this block: all, or one half (HALF: R is a multiple of 256,
  // so both halves are whole stages); s0 = the first one
  const int s0 = HALF ? half * (R / (2 * kBK)) : 0;
  const int nk = HALF ? R / (2 * kBK) : (R + kBK - 1) / kBK;
  const int nfull = HALF ? nk : R / kBK;   // full stages (all but a partial last one)

  // Buffer resources (base + byte count of each operand): being buffer (not
  // flat) loads, they leave the compiler's count of outstanding LDS reads
  // exact, so each MFMA waits only for its own fragments.
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)((uint32_t)M * (uint32_t)R), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsb =
      __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, (int)((uint32_t)N * (uint32_t)R), kRsrcWord3);
  // the 8 loads of A's (or B's) part of one full stage into slot sl. A
  // stage past the last full one (stage >= nfull) is loaded through a
  // resource of zero bytes: every lane is out of range, so nothing is read
  // from memory and zeros land in the slot, which no later read uses; the
  // loads still count in vmcnt, so the steady-state wait stays exact up to
  // the last stage.
  auto issue_a = [&](lds_u8* sl, int stage) {
    // wave-uniform; below 2^32 (operands are below 4 GiB), passed as int
    const int koffa = (int)((uint32_t)(s0 + stage) * kBK * (TA ? (uint32_t)M : 1u));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)A, (short)0, stage < nfull ? (int)((uint32_t)M * (uint32_t)R) : 0, kRsrcWord3);
    lds_u8* sa_ = sl + (8 * w) * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(sa_ + i * 1024), 16, (int)offa[i], koffa, 0, 0);
  };
  auto issue_b = [&](lds_u8* sl, int stage) {
    const int koffb = (int)((uint32_t)(s0 + stage) * kBK * (TB ? (uint32_t)N : 1u));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)B, (short)0, stage < nfull ? (int)((uint32_t)N * (uint32_t)R) : 0, kRsrcWord3);
    lds_u8* sb_ = sl + (8 * w) * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(sb_ + i * 1024), 16, (int)offb[i], koffb, 0, 0);
  };
  // any stage, including a partial last one (k past R zero-filled): A's
  // part (B = false) or B's part (B = true) into slot sl
  auto issue_any = [&](auto B_, lds_u8* sl, int stage) {
    constexpr bool IsB = decltype(B_)::value;
    if (stage < nfull) {
      if constexpr (IsB) issue_b(sl, stage);
      else issue_a(sl, stage);
      return;
    }
    constexpr bool T = IsB ? TB : TA;
    const int k0 = (s0 + stage) * kBK;
    lds_u8* dst = sl + (8 * w) * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lds_u8* d = dst + i * 1024;
      // first k of lane's 16 bytes (row layout) or lane's k-row (reduction-major)
      int lk;
      if constexpr (!T) {
        const int row = 8 * (8 * w + i) + (lane >> 3);
        lk = k0 + 16 * ((lane & 7) ^ swz(row));
      } else {
        lk = k0 + 4 * (8 * w + i) + (lane >> 4);
      }
      if (lk < R) {
        if constexpr (IsB)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (LDS_AS void*)d, 16, (int)offb[i],
                                                   (int)((uint32_t)k0 * (TB ? (uint32_t)N : 1u)), 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (LDS_AS void*)d, 16, (int)offa[i],
                                                   (int)((uint32_t)k0 * (TA ? (uint32_t)M : 1u)), 0, 0);
      } else {
        *(lds_u32x4*)(d + 16 * lane) = (u32x4){0, 0, 0, 0};
      }
    }
  };
  using IsA = std::false_type;
  using IsB = std::true_type;

  // ---- fragment reads: lane -> row (lane & 31); step h (0, 1) of a stage
  // takes logical chunks 4h + 2g and 4h + 2g + 1, g = lane >> 5. swz() of
  // every fragment row equals swz(lane & 31) (fragment rows start at
  // multiples of 32), so four per-lane offsets plus compile-time immediates
  // address every fragment of both buffers.
  const int frow = lane & 31, g = lane >> 5;
  const int fsw = swz(frow);
  int foff[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 2; ++j) foff[h][j] = frow * kBK + (((4 * h + 2 * g + j) ^ fsw) << 4);
  // Reduction-major operand: the part holds 128 k-rows of 256 output bytes.
  // A transposing LDS read (ds_read_b64_tr_b8) works on groups of 16 lanes:
  // lanes 2r and 2r+1 give the two 8-byte halves of a 16-byte row r
  // (r = 0..7), and lane i receives byte i of each of the 8 rows. Lane l's
  // group G = l / 16 covers outputs 16 (G % 2) .. + 15 of a 32-output block
  // and k-half G / 2; lane 2r + hh of the group points at k-row
  // 64 h + 32 (G / 2) + 8 t + r, byte 8 hh of the block's chunk, so read t
  // (t = 0..3) hands each lane k = 8 t .. 8 t + 7 of its k-half for output
  // (l & 31): the same 32 bytes the row layout reads. k-rows of one read
  // differ in (k & 7), so with the load swizzle (chunk ^ (k & 7)) they fall
  // in distinct banks. toff[f]: lane's offset for output block f; reads t
  // and steps h add 2048 t + 16384 h.
  int toff[4];
  {
    const int G = lane >> 4, j = lane & 15, r = j >> 1;
#pragma unroll
    for (int f4 = 0; f4 < 4; ++f4)
      toff[f4] = (32 * (G >> 1) + r) * 256 + (((2 * f4 + (G & 1)) ^ r) << 4) + 8 * (j & 1);
  }
  // wave-uniform fragment bases of A and B within their slots
  const int a_row0 = TA ? 128 * wm : 128 * wm * kBK;
  const int b_row0 = TB ? 128 * wn : 128 * wn * kBK;
  struct Frags {
    v8i a[4], b[4];
  };
  auto read_frag = [&](const lds_u8* p, int h) -> v8i {
    const u32x4 lo = *(const lds_u32x4*)(p + foff[h][0]);
    const u32x4 hi = *(const lds_u32x4*)(p + foff[h][1]);
    v8i v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
  };
  auto read_frag_t = [&](const lds_u8* p, int h, int f4) -> v8i {
    v8i v;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p + toff[f4] + 16384 * h + 2048 * tt));
      v[2 * tt] = x.x;
      v[2 * tt + 1] = x.y;
    }
    return v;
  };
  auto read_step = [&](const lds_u8* sla, const lds_u8* slb, int h, Frags& f) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if constexpr (TA) f.a[mi] = read_frag_t(sla + a_row0, h, mi);
      else f.a[mi] = read_frag(sla + a_row0 + 32 * mi * kBK, h);
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      if constexpr (TB) f.b[ni] = read_frag_t(slb + b_row0, h, ni);
      else f.b[ni] = read_frag(slb + b_row0 + 32 * ni * kBK, h);
    }
  };
  // LDS reads per step, spread evenly over its first 8 MFMAs below
  constexpr int kReadsPer = ((TA ? 4 : 2) + (TB ? 4 : 2)) / 2;

  v16f acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

  // Dequantisation 2^s, s = -(ba + bb), is applied to the FP32 sums in the
  // epilogue (exact power-of-two scaling). The MFMA could apply it through
  // its E8M0 operand scales instead, bit-identically wherever no product or
  // partial sum leaves the normal range, and save the epilogue's 256 ldexp
  // per lane; but the kernel runs at the chip's power limit, and the scaled
  // instruction measured ~1 % slower over the whole GEMM than the plain one
  // plus the ldexp. Literal zero scale operands select the plain
  // v_mfma_f32_32x32x64_f8f6f4 (no scaling).
  const int shift = -(sa->bias + sb->bias);
  auto mfma_all = [&](const Frags& f) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[ni], f.a[mi], acc[mi][ni], FB, FA,
                                                                       0, 0, 0, 0);
  };

  // Software pipeline. Stage s lives in A slot s % 2 and B slot s % 3; its
  // two MFMA steps use fr[0] (k-half 0) and fr[1] (k-half 1). On entry to
  // stage s, fr[0] holds its first half, and the loads in flight are B of
  // stage s+1, then A of stage s+1.
  //  step 2s:   read k-half 1 of stage s into fr[1]; issue B of stage s+2
  //             into the slot of stage s-1 (free since that stage's
  //             barrier); MFMAs on fr[0].
  //  step 2s+1: wait for stage s+1 (own loads by vmcnt: all but the last
  //             8, which are B of stage s+2; everyone's by the barrier,
  //             which also follows every wave's reads of stage s); issue A
  //             of stage s+2 into the A slot stage s freed; read k-half 0 of
  //             stage s+1 into fr[0]; MFMAs on fr[1].
  // Each step thus issues 8 of the stage's 16 loads: with all 16 in the
  // second step, the load path was busy for that whole step and held up
  // instruction issue (the step ran ~230 cycles over its 1024 of MFMAs; now
  // ~20-70).
  Frags fr[2];
  {
    if (nk > 0) {
      issue_any(IsA{}, a_slot<0>(), 0);
      issue_any(IsB{}, b_slot<0>(), 0);
    }
    if (nk > 1) {
      issue_any(IsA{}, a_slot<1>(), 1);
      issue_any(IsB{}, b_slot<1>(), 1);
    }
    // the accumulators are zeroed here, while the first loads are in
    // flight: left to the compiler, the 256 writes sat between the wait for
    // stage 0 and the first MFMA (~0.5 us per tile)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) asm volatile("" : "+a"(acc[mi][ni]));
    if (nk > 0) {
      if (nfull >= 3) wait_vmcnt<16>();  // stage 1 full: its 16 loads may stay in flight
      else wait_vmcnt<0>();              // a partial stage among the first ones: count not exact
      block_sync_lds();
      read_step(a_slot<0>(), b_slot<0>(), 0, fr[0]);
    }
  }
  // One stage in the steady state, with compile-time slots (J: the stage
  // index mod 6): the loads of A of stage s+2 and B of s+3 are issued (from
  // nothing when past the last stage, see issue_a). Hard scheduling fences
  // keep the order; the group hints interleave reads / loads with the MFMAs.
  auto stage_main = [&](auto J_, int s) {
    constexpr int J = decltype(J_)::value;
    read_step(a_slot<J>(), b_slot<J>(), 1, fr[1]);
    issue_b(b_slot<J + 2>(), s + 2);  // into the slot of stage s-1, free since its barrier
    mfma_all(fr[0]);
    static_for<16>([&](auto I_) {
      constexpr int i = decltype(I_)::value;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                         // MFMA
      if constexpr (i < 8) __builtin_amdgcn_sched_group_barrier(0x100, kReadsPer, 0);  // DS read
      if constexpr (i & 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);    // buffer load to LDS
    });
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<8>();   // A of stage s+1 landed (and B of s+1, issued before it); B of s+2 may fly
    block_sync_lds();  // everyone's loads landed, everyone's reads of stage s's slots done
    __builtin_amdgcn_sched_barrier(0);
    issue_a(a_slot<J>(), s + 2);
    read_step(a_slot<J + 1>(), b_slot<J + 1>(), 0, fr[0]);
    mfma_all(fr[1]);
    // one load per two MFMAs in either step: a stage's 64 KB of loads
    // issued in one step kept the load path busy for the whole step and
    // stalled instruction issue (that step ran ~230 cycles over its MFMAs)
    static_for<16>([&](auto I_) {
      constexpr int i = decltype(I_)::value;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                         // MFMA
      if constexpr (i < 8) __builtin_amdgcn_sched_group_barrier(0x100, kReadsPer, 0);  // DS read
      if constexpr (i & 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);    // buffer load to LDS
    });
    __builtin_amdgcn_sched_barrier(0);
  };
  // general stage (the last three when one of them is partial, or all of
  // them when there are fewer than three full stages):
  // bounds on every stage, all loads awaited in full, so the slots are
  // picked at run time; zero-filled parts of a partial stage are LDS
  // stores, made visible by the next barrier (block_sync_lds waits for
  // this wave's LDS accesses first)
  auto stage_any = [&](int s) {
    lds_u8* const as[2] = {a_slot<0>(), a_slot<1>()};
    lds_u8* const bs[3] = {b_slot<0>(), b_slot<1>(), b_slot<2>()};
    read_step(as[s & 1], bs[s % 3], 1, fr[1]);
    if (s + 2 < nk) issue_any(IsB{}, bs[(s + 2) % 3], s + 2);
    mfma_all(fr[0]);
    if (s + 1 < nk) {
      wait_vmcnt<0>();
      block_sync_lds();
      if (s + 2 < nk) issue_any(IsA{}, as[s & 1], s + 2);
      read_step(as[(s + 1) & 1], bs[(s + 1) % 3], 0, fr[0]);
    }
    mfma_all(fr[1]);
  };
  // Stages in the steady state: all of them when every stage is full (the
  // last ones load nothing, see issue_a), else those before the last three
  // full ones; whole rounds of six (slot indices repeat every six stages),
  // then the rest one by one. The stages after them take the general path.
  const int main_stages = (nk == nfull && nfull >= 3) ? nfull : (nfull > 3 ? nfull - 3 : 0);
  int s = 0;
  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  using J2 = std::integral_constant<int, 2>;
  using J3 = std::integral_constant<int, 3>;
  using J4 = std::integral_constant<int, 4>;
  using J5 = std::integral_constant<int, 5>;
  for (; s + 6 <= main_stages; s += 6) {
    stage_main(J0{}, s);
    stage_main(J1{}, s + 1);
    stage_main(J2{}, s + 2);
    stage_main(J3{}, s + 3);
    stage_main(J4{}, s + 4);
    stage_main(J5{}, s + 5);
  }
  const int rest = main_stages - s;
  if (rest > 0) stage_main(J0{}, s);
  if (rest > 1) stage_main(J1{}, s + 1);
  if (rest > 2) stage_main(J2{}, s + 2);
  if (rest > 3) stage_main(J3{}, s + 3);
  if (rest > 4) stage_main(J4{}, s + 4);
  s = main_stages;
  for (; s < nk; ++s) stage_any(s);
  wait_vmcnt<0>();
  block_sync_lds();

  if constexpr (HALF) {
    // partial sums out, 4 KB contiguous per store instruction (the thread
    // index through an empty asm keeps the addressing out of the k-loop)
    int te = t;
    asm volatile("" : "+v"(te));
    float* dst = part + 4 * te;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const v16f a = acc[mi][ni];
        float* d = dst + 4096 * (mi * 4 + ni);
        *(f32x4*)(d + 0) = __builtin_shufflevector(a, a, 0, 1, 2, 3);
        *(f32x4*)(d + 1024) = __builtin_shufflevector(a, a, 4, 5, 6, 7);
        *(f32x4*)(d + 2048) = __builtin_shufflevector(a, a, 8, 9, 10, 11);
        *(f32x4*)(d + 3072) = __builtin_shufflevector(a, a, 12, 13, 14, 15);
      }
    return;
  }

  // ---- epilogue, each wave on its own: 2^s (exact power-of-two scaling),
  // bf16 RNE, and the wave's 128 x 128 block of C written in four quarters
  // of 32 rows (accumulator row block mi). A quarter (32 rows x 256 bytes)
  // is staged row-major in the wave's own 8 KB of slot B2 and read back so
  // that 16 lanes hold one 256-byte row piece: a store instruction then
  // writes 4 rows x 256 bytes, whole cache lines (scattered 8-byte stores
  // had made HBM writes 5x the output size). The staging area is private
  // to the wave and one wave's LDS accesses are processed in order, so no
  // workgroup barrier is needed; the stores of one quarter drain while the
  // next is converted. 16-byte chunks of a staged row are XOR-swizzled by
  // (row & 15), which spreads both the 8-byte writes (32 rows x one chunk
  // per instruction) and the 16-byte reads over all banks.
  lds_u8* const wst = (lds_u8*)g_b2 + 8192 * w;
  // (the thread index is passed through an empty asm so that none of this
  // address arithmetic is hoisted above the k-loop, where registers are full)
  int te = t;
  asm volatile("" : "+v"(te));
  const int dl = te & 63, dc = dl & 15, dr = dl >> 4;  // read-back: chunk dc of rows dr + 4k
  int loff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) loff[kk] = (dr + 4 * kk) * 256 + ((dc ^ (dr + 4 * kk)) << 4);
  const int wsw = te & 15;                                            // frow & 15
  lds_u8* const wrow = wst + (te & 31) * 256 + 8 * ((te >> 5) & 1);  // row frow, half g
  const int col = n0 + 128 * wn + 8 * dc;
  const bool col_ok = col < N;
  const bool full_tile = m0 + kBM <= M && n0 + kBN <= N;
  // AMAX: max of the 15-bit magnitudes written, per quarter in cmax, then
  // reduced over the wave into the wave-uniform wmax
  uint32_t wmax = 0;
  auto quarter = [&](auto MI_, auto FULL_) {
    constexpr int mi = decltype(MI_)::value;
    constexpr bool FULL = decltype(FULL_)::value;
    u16x2 cmax = {0, 0};
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x2 lo = {ldexpf(acc[mi][ni][4 * q + 0], shift), ldexpf(acc[mi][ni][4 * q + 1], shift)};
        const f32x2 hi = {ldexpf(acc[mi][ni][4 * q + 2], shift), ldexpf(acc[mi][ni][4 * q + 3], shift)};
        const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
        const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
        // lane (frow, g) holds columns 32 ni + 8 q + 4 g .. + 3 of row frow:
        // half g of 16-byte chunk 4 ni + q
        *(lds_u32x2*)(wrow + (((4 * ni + q) ^ wsw) << 4)) = (u32x2){p0, p1};
        if constexpr (AMAX) {
          cmax = __builtin_elementwise_max(cmax, __builtin_bit_cast(u16x2, p0 & 0x7FFF7FFFu));
          cmax = __builtin_elementwise_max(cmax, __builtin_bit_cast(u16x2, p1 & 0x7FFF7FFFu));
        }
      }
      // one 32 x 32 block at a time, which bounds how many accumulators
      // are moved out of the accumulation registers at once
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (AMAX) {
      uint32_t r = cmax.x > cmax.y ? cmax.x : cmax.y;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)r, off, 64);
        r = o > r ? o : r;
      }
      r = __builtin_amdgcn_readfirstlane(r);
      wmax = r > wmax ? r : wmax;
    }
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = *(const lds_u32x4*)(wst + loff[k & 3] + (k >> 2) * 4096);
    const int row = m0 + 128 * wm + 32 * mi + dr;
    uint16_t* cp = C + (int64_t)row * N + col;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (FULL || (col_ok && row + 4 * k < M)) __builtin_nontemporal_store(v[k], (u32x4*)cp);
      cp += (int64_t)4 * N;
    }
  };
  auto all_quarters = [&](auto FULL_) {
    quarter(std::integral_constant<int, 0>{}, FULL_);
    quarter(std::integral_constant<int, 1>{}, FULL_);
    quarter(std::integral_constant<int, 2>{}, FULL_);
    quarter(std::integral_constant<int, 3>{}, FULL_);
  };
  if (full_tile) all_quarters(std::true_type{});
  else all_quarters(std::false_type{});
  // AMAX: rows past M and columns past N repeat valid rows / columns
  // (clamped operand rows), so the tile max is a max over real outputs;
  // one merge per wave
  if constexpr (AMAX) {
    if ((te & 63) == 0) {
      const unsigned long long v = (reduction_tag(s_out) << 16) | wmax;
      unsigned long long* word = (unsigned long long*)&s_out->gen_max;
      const unsigned long long seen = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (v > seen) atomicMax(word, v);
    }
    if (tile == 0 && te == 0) s_out->sat_count = 0u;
  }
}


// The same 256 x 256 tile on v_mfma_f32_16x16x128_f8f6f4 (row-layout A
// only: with a reduction-major A it needs more registers than the wave
// has). Loads, LDS slots, swizzles, the zero-byte resource past the last
// full stage and the per-wave epilogue are those of gemm_tile; the stage
// schedule differs: a stage's fragments are read during the previous
// stage, A of stage s+2 and B of stage s+3 are loaded into the slots of
// stage s (whose fragments are in registers by then), and one barrier
// opens each stage.
// tile: index of the output tile within the problem's tile grid.
// SPLIT (the tail-split kernel): half < 0 runs the whole tile as above;
// half = 0 or 1 takes that reduction half (R a multiple of 256) and stores
// its unscaled FP32 sums to `part` (65536 floats, float4 mi * 8 + ni of
// thread t at float offset 1024 (mi * 8 + ni) + 4 t) instead of the
// epilogue; gemm_tail_fixup_kernel<true> adds the two halves.
template <int FA, int FB, bool AMAX, bool TA, bool TB, bool SPLIT = false>
__device__ __forceinline__ void gemm_tile16(const GemmParams& p, int tile, fp8_scale_t* s_out, int half = -1,
                                            float* part = nullptr) {
  static_assert(!TA, "16 x 16 x 128 tile: row-layout A only");
  const uint8_t* __restrict__ A = p.A;
  const uint8_t* __restrict__ B = p.B;
  const fp8_scale_t* __restrict__ sa = p.sa;
  const fp8_scale_t* __restrict__ sb = p.sb;
  uint16_t* __restrict__ C = p.C;
  const int M = p.M, N = p.N, R = p.R, tiles_m = p.tiles_m, tiles_n = p.tiles_n;

  // ---- tile selection: XCD-contiguous ranges, grouped raster inside ----
  int m0, n0;
  tile_origin(tile, tiles_m, tiles_n, m0, n0);

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, scalar
  const int wm = w >> 1, wn = w & 1;

  // ---- loads: wave w fills 1 KB blocks 8w..8w+7 of the A and B parts of a
  // stage (a part is 32 KB). Row-layout operand: lane l of block b writes
  // row 8b + l/8 (an output index), LDS chunk l%8, which holds global chunk
  // (l%8) ^ swz(row) of that row's 128 k-bytes; rows past M / N read the
  // last valid row. Reduction-major operand: lane l of block b writes k-row
  // 4b + l/16, LDS chunk l%16 of that row's 256 output bytes, which holds
  // global chunk (l%16) ^ (krow & 7); chunks past M / N read the last valid
  // chunk, so the tile only ever holds real operand values. Operands are
  // below 4 GiB, so per-lane offsets are 32-bit; the stage offset is a
  // scalar (stage * 128 for rows, stage * 128 * M or N for reduction-major).
  // op_offset: product part p (laundered below) and added part c of lane's
  // offset for load i.
  auto op_offset = [&](auto T_, int i, int o0, int O, uint32_t& p, uint32_t& c) {
    if constexpr (!decltype(T_)::value) {
      const int row = 8 * (8 * w + i) + (lane >> 3);
      p = (uint32_t)min(o0 + row, O - 1) * (uint32_t)R;
      c = 16 * ((lane & 7) ^ swz(row));
    } else {
      const int krow = 4 * (8 * w + i) + (lane >> 4);
      p = (uint32_t)krow * (uint32_t)O;
      c = (uint32_t)min(o0 + 16 * ((lane & 15) ^ (krow & 7)), O - 16);
    }
  };
  using TAc = std::integral_constant<bool, TA>;
  using TBc = std::integral_constant<bool, TB>;
  // Lane's offset of load i: row layout, offa[i] (8 registers: rows are
  // clamped); reduction-major, the k-row of load i is 32 w + 4 i + l / 16,
  // so the offset is offa[i & 1] + 4 i M (the chunk swizzle k & 7 depends on
  // i only through i & 1), the second term scalar: 2 registers.
  uint32_t offa[8], offb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // 32-bit products, passed through an empty asm: fused into a 64-bit
    // multiply-add, each offset would occupy a register pair
    uint32_t pa, ca, pb, cb;
    op_offset(TAc{}, i, m0, M, pa, ca);
    op_offset(TBc{}, i, n0, N, pb, cb);
    asm volatile("" : "+v"(pa), "+v"(pb));
    offa[i] = pa + ca;
    offb[i] = pb + cb;
  }
  auto voffa = [&](int i) -> int { return (int)(TA ? offa[i & 1] : offa[i]); };
  auto voffb = [&](int i) -> int { return (int)(TB ? offb[i & 1] : offb[i]); };
  auto soffa = [&](int i) -> int { return TA ? 4 * (i & ~1) * M : 0; };
  auto soffb = [&](int i) -> int { return TB ? 4 * (i & ~1) * N : 0; };
  // stages of this block: all, or (SPLIT, half >= 0) one reduction half
  // (R is then a multiple of 256, so both halves are whole stages); s0 =
  // the first one. One k-loop serves both cases, so a tail-split launch
  // holds a single copy of it.
  const bool halfr = SPLIT && half >= 0;
  const int s0 = halfr ? half * (R / (2 * kBK)) : 0;
  const int nk = halfr ? R / (2 * kBK) : (R + kBK - 1) / kBK;
  const int nfull = halfr ? nk : R / kBK;   // full stages (all but a partial last one)

  // Buffer resources (base + byte count of each operand): being buffer (not
  // flat) loads, they leave the compiler's count of outstanding LDS reads
  // exact, so each MFMA waits only for its own fragments.
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)((uint32_t)M * (uint32_t)R), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsb =
      __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, (int)((uint32_t)N * (uint32_t)R), kRsrcWord3);
  // the 8 loads of A's (or B's) part of one full stage into slot sl. A
  // stage past the last full one (stage >= nfull) is loaded through a
  // resource of zero bytes: every lane is out of range, so nothing is read
  // from memory and zeros land in the slot, which no later read uses; the
  // loads still count in vmcnt, so the steady-state wait stays exact up to
  // the last stage.
  auto issue_a = [&](lds_u8* sl, int stage) {
    // wave-uniform; below 2^32 (operands are below 4 GiB), passed as int
    const int koffa = (int)((uint32_t)(s0 + stage) * kBK * (TA ? (uint32_t)M : 1u));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)A, (short)0, stage < nfull ? (int)((uint32_t)M * (uint32_t)R) : 0, kRsrcWord3);
    lds_u8* sa_ = sl + (8 * w) * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i)
    {
      const int vo = voffa(i), so = koffa + soffa(i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(sa_ + i * 1024), 16, vo, so, 0, 0);
    }
  };
  auto issue_b = [&](lds_u8* sl, int stage) {
    const int koffb = (int)((uint32_t)(s0 + stage) * kBK * (TB ? (uint32_t)N : 1u));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)B, (short)0, stage < nfull ? (int)((uint32_t)N * (uint32_t)R) : 0, kRsrcWord3);
    lds_u8* sb_ = sl + (8 * w) * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i)
    {
      const int vo = voffb(i), so = koffb + soffb(i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(sb_ + i * 1024), 16, vo, so, 0, 0);
    }
  };
  // any stage, including a partial last one (k past R zero-filled): A's
  // part (B = false) or B's part (B = true) into slot sl
  auto issue_any = [&](auto B_, lds_u8* sl, int stage) {
    constexpr bool IsB = decltype(B_)::value;
    if (stage < nfull) {
      if constexpr (IsB) issue_b(sl, stage);
      else issue_a(sl, stage);
      return;
    }
    constexpr bool T = IsB ? TB : TA;
    const int k0 = (s0 + stage) * kBK;
    lds_u8* dst = sl + (8 * w) * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lds_u8* d = dst + i * 1024;
      // first k of lane's 16 bytes (row layout) or lane's k-row (reduction-major)
      int lk;
      if constexpr (!T) {
        const int row = 8 * (8 * w + i) + (lane >> 3);
        lk = k0 + 16 * ((lane & 7) ^ swz(row));
      } else {
        lk = k0 + 4 * (8 * w + i) + (lane >> 4);
      }
      if (lk < R) {
        if constexpr (IsB)
        {
          const int vo = voffb(i), so = (int)((uint32_t)k0 * (TB ? (uint32_t)N : 1u)) + soffb(i);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (LDS_AS void*)d, 16, vo, so, 0, 0);
        }
        else
        {
          const int vo = voffa(i), so = (int)((uint32_t)k0 * (TA ? (uint32_t)M : 1u)) + soffa(i);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (LDS_AS void*)d, 16, vo, so, 0, 0);
        }
      } else {
        *(lds_u32x4*)(d + 16 * lane) = (u32x4){0, 0, 0, 0};
      }
    }
  };
  using IsA = std::false_type;
  using IsB = std::true_type;

  // ---- fragment reads. v_mfma_f32_16x16x128_f8f6f4 takes from lane l row
  // l % 16 of a 16-row block and k bytes 32 G .. 32 G + 31 (G = l / 16) of
  // it, for either operand (lane layout checked on the device with an
  // in-bounds probe), so one MFMA consumes a whole stage of k = 128.
  // Row-layout operand: the fragment of block m (rows 16 m .. 16 m + 15 of
  // the wave's 128) is two 16-byte reads, logical chunks 2 G and 2 G + 1 of
  // row 16 m + (l % 16); swz() of that row is swz(l % 16), so two per-lane
  // offsets plus immediates (2048 m) address every fragment.
  const int fr16 = lane & 15, fG = lane >> 4;
  int foff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) foff[j] = fr16 * kBK + (((2 * fG + j) ^ swz(fr16)) << 4);
  // Reduction-major operand: the part holds 128 k-rows of 256 output bytes
  // (chunk c = outputs 16 c .. 16 c + 15, stored at chunk c ^ (k & 7)). A
  // transposing LDS read (ds_read_b64_tr_b8) works on groups of 16 lanes:
  // lanes 2r and 2r+1 give the two 8-byte halves of a 16-byte row r
  // (r = 0..7), and lane i receives byte i of each of the 8 rows. Group G =
  // l / 16 takes k-rows 32 G + 8 t + r (t = 0..3, one read each), so lane l
  // gets output l % 16 of the block with k = 32 G .. 32 G + 31, the bytes
  // the row layout hands it. The wave's block m of B is chunk 8 wn + m,
  // stored at 8 wn + (m ^ r) in those rows; read t adds 2048 t. The rows of
  // one read differ in k & 7, so they fall in distinct banks.
  // toff(m) = tbase + ((m ^ r) << 4) = tbase + ((m << 4) ^ trx): two
  // registers, the XOR done per fragment (with trx passed through an empty
  // asm once per stage, so eight precomputed offsets are not held)
  const int tbase = (32 * (lane >> 4) + ((lane & 15) >> 1)) * 256 + 8 * (lane & 1);
  const int trx = ((lane & 15) >> 1) << 4;
  // wave-uniform fragment bases of A and B within their slots
  const int a_row0 = TA ? 128 * wm : 128 * wm * kBK;
  const int b_row0 = TB ? 128 * wn : 128 * wn * kBK;
  // fragment of block m of an operand whose wave base in its slot is p
  // (rx: trx, passed through an empty asm by the caller)
  auto frag = [&](auto T_, const lds_u8* p, auto M_, int rx) -> v8i {
    constexpr int m = decltype(M_)::value;
    v8i v;
    if constexpr (!decltype(T_)::value) {
      const u32x4 lo = *(const lds_u32x4*)(p + foff[0] + 2048 * m);
      const u32x4 hi = *(const lds_u32x4*)(p + foff[1] + 2048 * m);
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    } else {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p + tbase + ((m << 4) ^ rx) + 2048 * tt));
        v[2 * tt] = x.x;
        v[2 * tt + 1] = x.y;
      }
    }
    return v;
  };
  using TAc2 = std::integral_constant<bool, TA>;
  using TBc2 = std::integral_constant<bool, TB>;
  constexpr int kReadsA = TA ? 4 : 2, kReadsB = TB ? 4 : 2;  // LDS reads per fragment

  // accumulators: block (mi, ni) of 16 x 16 (lane l holds output row
  // 16 mi + l % 16, columns 16 ni + 4 (l / 16) .. + 3)
  f32x4 acc[8][8];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int ni = 0; ni < 8; ++ni)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[mi][ni][v] = 0.0f;

  // Dequantisation 2^s, s = -(ba + bb), is applied to the FP32 sums in the
  // epilogue (exact power-of-two scaling). The MFMA could apply it through
  // its E8M0 operand scales instead, bit-identically wherever no product or
  // partial sum leaves the normal range, and save the epilogue's ldexp; but
  // the kernel runs at the chip's power limit, and the scaled instruction
  // measured ~1 % slower over the whole GEMM than the plain one plus the
  // ldexp. Literal zero scale operands select the plain instruction.
  const int shift = -(sa->bias + sb->bias);
  auto mfma = [&](const v8i& b, const v8i& a, f32x4& c) {
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, FB, FA, 0, 0, 0, 0);
  };

  // Fragments in registers (P = parity of the stage): A blocks 0..5 in
  // fa[0..5], A blocks 6, 7 in fa67[P][0..1], B blocks 0..3 in fb[0..3], B
  // blocks 4..7 in fb47[P][0..3] (176 registers).
  v8i fa[6], fa67[2][2], fb[4], fb47[2][4];
  auto read_all = [&](const lds_u8* pa, const lds_u8* pb) {  // a whole stage into set 0
    int rx = trx;
    asm volatile("" : "+v"(rx));
    static_for<6>([&](auto M_) { fa[decltype(M_)::value] = frag(TAc2{}, pa, M_, rx); });
    fa67[0][0] = frag(TAc2{}, pa, std::integral_constant<int, 6>{}, rx);
    fa67[0][1] = frag(TAc2{}, pa, std::integral_constant<int, 7>{}, rx);
    static_for<4>([&](auto N_) { fb[decltype(N_)::value] = frag(TBc2{}, pb, N_, rx); });
    static_for<4>([&](auto N_) {
      fb47[0][decltype(N_)::value] = frag(TBc2{}, pb, std::integral_constant<int, 4 + decltype(N_)::value>{}, rx);
    });
  };
  {
    if (nk > 0) {
      issue_any(IsA{}, a_slot<0>(), 0);
      issue_any(IsB{}, b_slot<0>(), 0);
    }
    if (nk > 1) {
      issue_any(IsA{}, a_slot<1>(), 1);
      issue_any(IsB{}, b_slot<1>(), 1);
    }
    if (nk > 2) issue_any(IsB{}, b_slot<2>(), 2);
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) asm volatile("" : "+a"(acc[mi][ni]));
    if (nk > 0) {
      if (nfull >= 3) wait_vmcnt<24>();
      else wait_vmcnt<0>();
      block_sync_lds();
      read_all(a_slot<0>() + a_row0, b_slot<0>() + b_row0);
    }
  }
  // 2 (or 1) of the 8 loads of A's (B's) part of a full stage, from load i0
  auto issue_a2 = [&](lds_u8* sl, int stage, int i0) {
    const int koffa = (int)((uint32_t)(s0 + stage) * kBK * (TA ? (uint32_t)M : 1u));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)A, (short)0, stage < nfull ? (int)((uint32_t)M * (uint32_t)R) : 0, kRsrcWord3);
    lds_u8* sa_ = sl + (8 * w) * 1024;
#pragma unroll
    for (int i = i0; i < i0 + 2; ++i)
    {
      const int vo = voffa(i), so = koffa + soffa(i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(sa_ + i * 1024), 16, vo, so, 0, 0);
    }
  };
  auto issue_b1 = [&](lds_u8* sl, int stage, int i) {
    const int koffb = (int)((uint32_t)(s0 + stage) * kBK * (TB ? (uint32_t)N : 1u));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)B, (short)0, stage < nfull ? (int)((uint32_t)N * (uint32_t)R) : 0, kRsrcWord3);
    const int vo = voffb(i), so = koffb + soffb(i);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(sl + (8 * w) * 1024 + i * 1024), 16, vo, so, 0, 0);
  };
  // hint sequence for a region of NM MFMAs, NR LDS reads and NL loads
  auto hints = [&](auto NM_, auto NR_, auto NL_) {
    constexpr int NM = decltype(NM_)::value, NR = decltype(NR_)::value, NL = decltype(NL_)::value;
    static_for<NM>([&](auto I_) {
      constexpr int i = decltype(I_)::value;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      constexpr int r = (NR * (i + 1)) / NM - (NR * i) / NM;
      if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // DS read
      constexpr int l = (NL * (i + 1)) / NM - (NL * i) / NM;
      if constexpr (l > 0) __builtin_amdgcn_sched_group_barrier(0x020, l, 0);  // buffer load to LDS
    });
    __builtin_amdgcn_sched_barrier(0);
  };
  using I1c = std::integral_constant<int, 1>;
  using I2c = std::integral_constant<int, 2>;
  using I4c = std::integral_constant<int, 4>;
  using I8c = std::integral_constant<int, 8>;
  // One stage in the steady state, with compile-time slots and register
  // sets (J: the stage index mod 6). Each row / column block is a region
  // between hard scheduling fences, so a fragment register is refilled only
  // after the MFMAs that read it.
  auto stage_main = [&](auto J_, int s) {
    constexpr int J = decltype(J_)::value, P = J & 1, Q = P ^ 1;
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<8>();   // A and B of stage s+1 landed; B of stage s+2 may fly
    block_sync_lds();  // everyone's loads landed, everyone's reads of stage s's slots done
    __builtin_amdgcn_sched_barrier(0);
    const lds_u8* na = a_slot<J + 1>() + a_row0;
    const lds_u8* nb = b_slot<J + 1>() + b_row0;
    int rx = trx;
    asm volatile("" : "+v"(rx));
    auto B_ = [&](auto N_) -> const v8i& {
      constexpr int n = decltype(N_)::value;
      if constexpr (n < 4) return fb[n];
      else return fb47[P][n - 4];
    };
    // row blocks 0..3 (8 MFMAs each): A loads; reads of A block mi - 1 in
    // place and of the double-buffered blocks (B 4..7, A 6, 7)
    static_for<4>([&](auto MI_) {
      constexpr int mi = decltype(MI_)::value;
      issue_a2(a_slot<J>(), s + 2, 2 * mi);
      fb47[Q][mi] = frag(TBc2{}, nb, std::integral_constant<int, 4 + mi>{}, rx);
      if constexpr (mi >= 2) fa67[Q][mi - 2] = frag(TAc2{}, na, std::integral_constant<int, 4 + mi>{}, rx);
      if constexpr (mi >= 1) fa[mi - 1] = frag(TAc2{}, na, std::integral_constant<int, mi - 1>{}, rx);
      static_for<8>([&](auto N_) { mfma(B_(N_), fa[mi], acc[mi][decltype(N_)::value]); });
      constexpr int nr = kReadsB + (mi >= 2 ? kReadsA : 0) + (mi >= 1 ? kReadsA : 0);
      hints(I8c{}, std::integral_constant<int, nr>{}, I2c{});
    });
    // column pairs over rows 4, 5: B loads; A block 3 in place
    static_for<4>([&](auto C_) {
      constexpr int c = decltype(C_)::value;
      issue_b1(b_slot<J>(), s + 3, c);
      if constexpr (c == 0) fa[3] = frag(TAc2{}, na, std::integral_constant<int, 3>{}, rx);
      static_for<2>([&](auto D_) {
        using Nc = std::integral_constant<int, 2 * c + decltype(D_)::value>;
        mfma(B_(Nc{}), fa[4], acc[4][Nc::value]);
        mfma(B_(Nc{}), fa[5], acc[5][Nc::value]);
      });
      hints(I4c{}, std::integral_constant<int, c == 0 ? kReadsA : 0>{}, I1c{});
    });
    // column pairs over rows 6, 7: B loads; A blocks 4, 5 in place (pair 0),
    // B blocks 0, 1 (pair 1) and 2, 3 (pair 2) in place; none in the last
    static_for<4>([&](auto C_) {
      constexpr int c = decltype(C_)::value;
      issue_b1(b_slot<J>(), s + 3, 4 + c);
      if constexpr (c == 0) {
        fa[4] = frag(TAc2{}, na, std::integral_constant<int, 4>{}, rx);
        fa[5] = frag(TAc2{}, na, std::integral_constant<int, 5>{}, rx);
      } else if constexpr (c <= 2) {
        fb[2 * c - 2] = frag(TBc2{}, nb, std::integral_constant<int, 2 * c - 2>{}, rx);
        fb[2 * c - 1] = frag(TBc2{}, nb, std::integral_constant<int, 2 * c - 1>{}, rx);
      }
      static_for<2>([&](auto D_) {
        using Nc = std::integral_constant<int, 2 * c + decltype(D_)::value>;
        mfma(B_(Nc{}), fa67[P][0], acc[6][Nc::value]);
        mfma(B_(Nc{}), fa67[P][1], acc[7][Nc::value]);
      });
      hints(I4c{}, std::integral_constant<int, c == 0 ? 2 * kReadsA : (c <= 2 ? 2 * kReadsB : 0)>{}, I1c{});
    });
  };
  // general stage (the last three when one of them is partial, or all of
  // them when there are fewer than three full stages): bounds on every
  // stage, all loads awaited in full, the slots picked at run time, the
  // stage's fragments read into set 0 after its barrier, and the loads into
  // its slots issued after a second one; zero-filled parts of a partial
  // stage are LDS stores, made visible by the next barrier (block_sync_lds
  // waits for this wave's LDS accesses first)
  auto stage_any = [&](int s) {
    lds_u8* const as[2] = {a_slot<0>(), a_slot<1>()};
    lds_u8* const bs[3] = {b_slot<0>(), b_slot<1>(), b_slot<2>()};
    wait_vmcnt<0>();
    block_sync_lds();
    read_all(as[s & 1] + a_row0, bs[s % 3] + b_row0);
    block_sync_lds();
    if (s + 2 < nk) issue_any(IsA{}, as[s & 1], s + 2);
    if (s + 3 < nk) issue_any(IsB{}, bs[s % 3], s + 3);
    auto A0 = [&](auto M_) -> const v8i& {
      constexpr int m = decltype(M_)::value;
      if constexpr (m < 6) return fa[m];
      else return fa67[0][m - 6];
    };
    auto B0 = [&](auto N_) -> const v8i& {
      constexpr int n = decltype(N_)::value;
      if constexpr (n < 4) return fb[n];
      else return fb47[0][n - 4];
    };
    static_for<8>([&](auto M_) {
      static_for<8>([&](auto N_) { mfma(B0(N_), A0(M_), acc[decltype(M_)::value][decltype(N_)::value]); });
    });
  };
  // Stages in the steady state: all of them when every stage is full (the
  // last ones load nothing, see issue_a), else those before the last three
  // full ones; whole rounds of six (slot indices repeat every six stages),
  // then the rest one by one. The stages after them take the general path.
  const int main_stages = (nk == nfull && nfull >= 3) ? nfull : (nfull > 3 ? nfull - 3 : 0);
  int s = 0;
  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  using J2 = std::integral_constant<int, 2>;
  using J3 = std::integral_constant<int, 3>;
  using J4 = std::integral_constant<int, 4>;
  using J5 = std::integral_constant<int, 5>;
  for (; s + 6 <= main_stages; s += 6) {
    stage_main(J0{}, s);
    stage_main(J1{}, s + 1);
    stage_main(J2{}, s + 2);
    stage_main(J3{}, s + 3);
    stage_main(J4{}, s + 4);
    stage_main(J5{}, s + 5);
  }
  const int rest = main_stages - s;
  if (rest > 0) stage_main(J0{}, s);
  if (rest > 1) stage_main(J1{}, s + 1);
  if (rest > 2) stage_main(J2{}, s + 2);
  if (rest > 3) stage_main(J3{}, s + 3);
  if (rest > 4) stage_main(J4{}, s + 4);
  s = main_stages;
  for (; s < nk; ++s) stage_any(s);
  wait_vmcnt<0>();
  block_sync_lds();

  if (halfr) {
    // partial sums out in register order (float4 mi * 8 + ni of thread t at
    // float offset 1024 (mi * 8 + ni) + 4 t), 4 KB contiguous per store
    // instruction; the thread index through an empty asm keeps the
    // addressing out of the k-loop
    int te = t;
    asm volatile("" : "+v"(te));
    float* dst = part + 4 * te;
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) *(f32x4*)(dst + 1024 * (mi * 8 + ni)) = acc[mi][ni];
    return;
  }

  // ---- epilogue, each wave on its own: 2^s (exact power-of-two scaling),
  // bf16 RNE, and the wave's 128 x 128 block of C written in four quarters
  // of 32 rows (accumulator row blocks 2q, 2q + 1). A quarter (32 rows x 256 bytes)
  // is staged row-major in the wave's own 8 KB of slot B2 and read back so
  // that 16 lanes hold one 256-byte row piece: a store instruction then
  // writes 4 rows x 256 bytes, whole cache lines (scattered 8-byte stores
  // had made HBM writes 5x the output size). The staging area is private
  // to the wave and one wave's LDS accesses are processed in order, so no
  // workgroup barrier is needed; the stores of one quarter drain while the
  // next is converted. 16-byte chunks of a staged row are XOR-swizzled by
  // (row & 15), which spreads both the 8-byte writes (32 rows x one chunk
  // per instruction) and the 16-byte reads over all banks.
  lds_u8* const wst = (lds_u8*)g_b2 + 8192 * w;
  // (the thread index is passed through an empty asm so that none of this
  // address arithmetic is hoisted above the k-loop, where registers are full)
  int te = t;
  asm volatile("" : "+v"(te));
  const int dl = te & 63, dc = dl & 15, dr = dl >> 4;  // read-back: chunk dc of rows dr + 4k
  int loff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) loff[kk] = (dr + 4 * kk) * 256 + ((dc ^ (dr + 4 * kk)) << 4);
  // lane (r16 = l % 16, G = l / 16) writes row 16 mm + r16 of a quarter
  // (mm = row block within it), half G & 1 of chunks 2 ni + (G >> 1)
  const int wsw = te & 15;                                                   // r16 (row & 15)
  lds_u8* const wrow = wst + (te & 15) * 256 + 8 * ((te >> 4) & 1);         // row r16, half G & 1
  const int wg2 = (te >> 5) & 1;                                            // G >> 1
  const int col = n0 + 128 * wn + 8 * dc;
  const bool col_ok = col < N;
  const bool full_tile = m0 + kBM <= M && n0 + kBN <= N;
  // AMAX: max of the 15-bit magnitudes written, per quarter in cmax, then
  // reduced over the wave into the wave-uniform wmax
  uint32_t wmax = 0;
  auto quarter = [&](auto MI_, auto FULL_) {
    constexpr int mi = decltype(MI_)::value;  // quarter index: row blocks 2 mi, 2 mi + 1
    constexpr bool FULL = decltype(FULL_)::value;
    u16x2 cmax = {0, 0};
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) {
        const f32x4 a = acc[2 * mi + mm][ni];
        const f32x2 lo = {ldexpf(a[0], shift), ldexpf(a[1], shift)};
        const f32x2 hi = {ldexpf(a[2], shift), ldexpf(a[3], shift)};
        const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
        const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
        // columns 16 ni + 4 G .. + 3 of row 16 mm + r16
        *(lds_u32x2*)(wrow + 4096 * mm + (((2 * ni + wg2) ^ wsw) << 4)) = (u32x2){p0, p1};
        if constexpr (AMAX) {
          cmax = __builtin_elementwise_max(cmax, __builtin_bit_cast(u16x2, p0 & 0x7FFF7FFFu));
          cmax = __builtin_elementwise_max(cmax, __builtin_bit_cast(u16x2, p1 & 0x7FFF7FFFu));
        }
        // a few blocks at a time, which bounds how many accumulators are
        // moved out of the accumulation registers at once
        if (ni % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (AMAX) {
      uint32_t r = cmax.x > cmax.y ? cmax.x : cmax.y;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)r, off, 64);
        r = o > r ? o : r;
      }
      r = __builtin_amdgcn_readfirstlane(r);
      wmax = r > wmax ? r : wmax;
    }
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = *(const lds_u32x4*)(wst + loff[k & 3] + (k >> 2) * 4096);
    const int row = m0 + 128 * wm + 32 * mi + dr;
    uint16_t* cp = C + (int64_t)row * N + col;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (FULL || (col_ok && row + 4 * k < M)) __builtin_nontemporal_store(v[k], (u32x4*)cp);
      cp += (int64_t)4 * N;
    }
  };
  auto all_quarters = [&](auto FULL_) {
    quarter(std::integral_constant<int, 0>{}, FULL_);
    quarter(std::integral_constant<int, 1>{}, FULL_);
    quarter(std::integral_constant<int, 2>{}, FULL_);
    quarter(std::integral_constant<int, 3>{}, FULL_);
  };
  if (full_tile) all_quarters(std::true_type{});
  else all_quarters(std::false_type{});
  // AMAX: rows past M and columns past N repeat valid rows / columns
  // (clamped operand rows), so the tile max is a max over real outputs;
  // one merge per wave
  if constexpr (AMAX) {
    if ((te & 63) == 0) {
      const unsigned long long v = (reduction_tag(s_out) << 16) | wmax;
      unsigned long long* word = (unsigned long long*)&s_out->gen_max;
      const unsigned long long seen = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (v > seen) atomicMax(word, v);
    }
    if (tile == 0 && te == 0) s_out->sat_count = 0u;
  }
}

// Which tile body a kernel uses: the 16 x 16 x 128 one wherever A has
// one row per output index, except the fused-amax variant with a
// reduction-major B (that combination needs more registers than the wave
// has and is used by no training path); the 32 x 32 x 64 one otherwise.
// Layouts that share a body give identical bits; the two bodies round
// their FP32 partial sums at different points (rarely one bf16 ulp apart).
constexpr bool k128_tile(bool ta, bool tb, bool amax) { return !ta && !(amax && tb); }

// One GEMM: one block per output tile.
template <int FA, int FB, bool AMAX, bool TA, bool TB>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(GemmParams p, fp8_scale_t* s_out) {
  if constexpr (k128_tile(TA, TB, AMAX)) gemm_tile16<FA, FB, AMAX, TA, TB>(p, (int)blockIdx.x, s_out);
  else gemm_tile<FA, FB, AMAX, TA, TB>(p, (int)blockIdx.x, s_out);
}

// Two GEMMs in one launch: blocks below p0's tile count take p0's tiles,
// the rest p1's, each with the code of its own variant (the first GEMM's
// tiles are dispatched first). A block does exactly what the single-GEMM
// kernel's block for that tile does, so the results are bit-identical;
// one launch instead of two saves the launch ramp and lets the second
// GEMM's tiles fill the first one's tail. Instantiated for the linear
// backward: dgrad (E5M2 dy8 x E4M3 w8, both one row per output index: the
// 16 x 16 x 128 body) and wgrad (E4M3 x8 x E5M2 dy8, both reduction-major:
// the 32 x 32 x 64 body).
template <int FA0, int FB0, bool TA0, bool TB0, int FA1, int FB1, bool TA1, bool TB1>
__global__ __launch_bounds__(kThreads, 1) void gemm_pair_kernel(GemmParams p0, GemmParams p1) {
  const int b = (int)blockIdx.x, n0 = p0.tiles_m * p0.tiles_n;
  if (b < n0) {
    if constexpr (k128_tile(TA0, TB0, false)) gemm_tile16<FA0, FB0, false, TA0, TB0>(p0, b, nullptr);
    else gemm_tile<FA0, FB0, false, TA0, TB0>(p0, b, nullptr);
  } else {
    if constexpr (k128_tile(TA1, TB1, false)) gemm_tile16<FA1, FB1, false, TA1, TB1>(p1, b - n0, nullptr);
    else gemm_tile<FA1, FB1, false, TA1, TB1>(p1, b - n0, nullptr);
  }
}

// Tail split: tiles [0, nfull) as in gemm_nt_kernel (same body, same
// bits); each of the ntail tiles after them (the last, partial wave:
// ntail <= half the CUs) is taken by two blocks, one per reduction half,
// which store FP32 partial sums to part (two 65536-float slots per tail
// tile). The last wave then runs 2 * ntail half-length blocks instead of
// ntail whole ones. The 16 x 16 x 128 body takes both roles through one
// k-loop (the half a run-time argument): two inlined copies of it would
// not fit the registers together.
template <int FA, int FB, bool TA, bool TB>
__global__ __launch_bounds__(kThreads, 1) void gemm_tailsplit_kernel(GemmParams p, int nfull, float* part) {
  const int b = (int)blockIdx.x;
  if constexpr (k128_tile(TA, TB, false)) {
    const bool tail = b >= nfull;
    const int u = b - nfull, j = u >> 1;
    gemm_tile16<FA, FB, false, TA, TB, true>(p, tail ? nfull + j : b, nullptr, tail ? (u & 1) : -1,
                                             tail ? part + (size_t)(2 * j + (u & 1)) * 65536 : nullptr);
  } else if (b < nfull) {
    gemm_tile<FA, FB, false, TA, TB>(p, b, nullptr);
  } else {
    const int u = b - nfull, j = u >> 1;
    gemm_tile<FA, FB, false, TA, TB, true>(p, nfull + j, nullptr, u & 1, part + (size_t)(2 * j + (u & 1)) * 65536);
  }
}

// C tiles of the tail: half 0 + half 1 (in that order, FP32), times
// 2^-(ba + bb), bf16 RNE; staged in LDS and written in whole rows as the
// GEMM epilogue does. Block j finishes tail tile nfull + j. K128: the
// partials are in the 16 x 16 x 128 body's register order, else in the
// 32 x 32 x 64 one's.
template <bool K128>
__global__ __launch_bounds__(kThreads, 1) void gemm_tail_fixup_kernel(GemmParams p, int nfull, const float* part) {
  const int j = (int)blockIdx.x;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), wm = w >> 1, wn = w & 1;
  int m0, n0;
  tile_origin(nfull + j, p.tiles_m, p.tiles_n, m0, n0);
  const int M = p.M, N = p.N;
  const int shift = -(p.sa->bias + p.sb->bias);
  const float* h0 = part + (size_t)(2 * j) * 65536 + 4 * t;
  const float* h1 = h0 + 65536;
  if constexpr (K128) {
    // 16 x 16 x 128 tiles: float4 mi * 8 + ni of thread t holds row
    // 128 wm + 16 mi + (l % 16), columns 128 wn + 16 ni + 4 (l / 16) .. + 3
    const int r16 = lane & 15, G = lane >> 4;
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
      const int row = 128 * wm + 16 * mi + r16;
      lds_u8* crow = c_region(row >> 6) + (row & 63) * 512;
      f32x4 a[8], b[8];
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) {
        a[ni] = __builtin_nontemporal_load((const f32x4*)(h0 + 1024 * (mi * 8 + ni)));
        b[ni] = __builtin_nontemporal_load((const f32x4*)(h1 + 1024 * (mi * 8 + ni)));
      }
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) {
        const f32x4 sum = a[ni] + b[ni];  // half 0 + half 1
        const f32x2 lo = {ldexpf(sum.x, shift), ldexpf(sum.y, shift)};
        const f32x2 hi = {ldexpf(sum.z, shift), ldexpf(sum.w, shift)};
        const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
        const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
        const int chunk = 16 * wn + 2 * ni + (G >> 1);
        *(lds_u32x2*)(crow + ((chunk ^ (row & 31)) << 4) + 8 * (G & 1)) = (u32x2){p0, p1};
      }
    }
  } else {
  // 32 x 32 x 64 tiles: float4 (mi * 4 + ni) * 4 + q of thread t holds row
  // 128 wm + 32 mi + (l % 32), columns 128 wn + 32 ni + 8 q + 4 (l / 32) .. + 3
  const int frow = lane & 31, g = lane >> 5;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int row = 128 * wm + 32 * mi + frow;
    lds_u8* crow = c_region(2 * wm + (mi >> 1)) + (row & 63) * 512;
    f32x4 a[16], b[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      a[k] = __builtin_nontemporal_load((const f32x4*)(h0 + 1024 * (mi * 16 + k)));
      b[k] = __builtin_nontemporal_load((const f32x4*)(h1 + 1024 * (mi * 16 + k)));
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 sum = a[ni * 4 + q] + b[ni * 4 + q];  // half 0 + half 1
        const f32x2 lo = {ldexpf(sum.x, shift), ldexpf(sum.y, shift)};
        const f32x2 hi = {ldexpf(sum.z, shift), ldexpf(sum.w, shift)};
        const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
        const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
        const int chunk = 16 * wn + 4 * ni + q;
        *(lds_u32x2*)(crow + ((chunk ^ (row & 31)) << 4) + 8 * g) = (u32x2){p0, p1};
      }
    }
  }
  }
  __syncthreads();
  // drain as the GEMM epilogue: lane t takes 16-byte chunk c = t % 32 of
  // rows r0 + 8k (r0 = t / 32) of each 64-row region
  const int c = t & 31, r0 = t >> 5;
  const bool col_ok = n0 + 8 * c < N;
#pragma unroll
  for (int reg = 0; reg < 4; ++reg) {
    const lds_u8* src = c_region(2 * (reg >> 1) + (reg & 1));
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = r0 + 8 * k;  // row within the 64-row region
      const u32x4 v = *(const lds_u32x4*)(src + r * 512 + ((c ^ (r & 31)) << 4));
      const int grow = m0 + 64 * reg + r;
      if (col_ok && grow < M) __builtin_nontemporal_store(v, (u32x4*)(p.C + (int64_t)grow * N + n0 + 8 * c));
    }
  }
}

inline GemmParams make_params(const uint8_t* A, const fp8_scale_t* sa, const uint8_t* B, const fp8_scale_t* sb,
                              int64_t M, int64_t N, int64_t R, void* C) {
  GemmParams p;
  p.A = A;
  p.B = B;
  p.sa = sa;
  p.sb = sb;
  p.C = (uint16_t*)C;
  p.M = (int)M;
  p.N = (int)N;
  p.R = (int)R;
  p.tiles_m = (int)((M + kBM - 1) / kBM);
  p.tiles_n = (int)((N + kBN - 1) / kBN);
  return p;
}

template <int FA, int FB, bool AMAX, bool TA, bool TB>
hipError_t launch_typed(const uint8_t* A, const fp8_scale_t* sa, const uint8_t* B, const fp8_scale_t* sb,
                        int64_t M, int64_t N, int64_t R, void* C, hipStream_t st, fp8_scale_t* s_out) {
  const GemmParams p = make_params(A, sa, B, sb, M, N, R, C);
  hipLaunchKernelGGL((gemm_nt_kernel<FA, FB, AMAX, TA, TB>), dim3(p.tiles_m * p.tiles_n), dim3(kThreads), 0, st,
                     p, s_out);
  return hipGetLastError();
}

// CUs of the current device (cached per device)
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <bool TA, bool TB>
hipError_t launch_tailsplit(const uint8_t* A, const fp8_scale_t* sa, const uint8_t* B, const fp8_scale_t* sb,
                            int64_t M, int64_t N, int64_t R, void* C, const TailSplit& ts, float* part,
                            hipStream_t st) {
  constexpr int E4 = FP8_E4M3;
  const GemmParams p = make_params(A, sa, B, sb, M, N, R, C);
  hipLaunchKernelGGL((gemm_tailsplit_kernel<E4, E4, TA, TB>), dim3(ts.nfull + 2 * ts.ntail), dim3(kThreads), 0, st,
                     p, ts.nfull, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_tail_fixup_kernel<k128_tile(TA, TB, false)>, dim3(ts.ntail), dim3(kThreads), 0, st, p, ts.nfull,
                     (const float*)part);
  return hipGetLastError();
}

template <int FA, int FB>
hipError_t launch_layouts(const uint8_t* A, bool ta, const fp8_scale_t* sa, const uint8_t* B, bool tb,
                          const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R, void* C, hipStream_t st) {
  if (!ta && !tb) return launch_typed<FA, FB, false, false, false>(A, sa, B, sb, M, N, R, C, st, nullptr);
  if (!ta && tb) return launch_typed<FA, FB, false, false, true>(A, sa, B, sb, M, N, R, C, st, nullptr);
  if (ta && !tb) return launch_typed<FA, FB, false, true, false>(A, sa, B, sb, M, N, R, C, st, nullptr);
  return launch_typed<FA, FB, false, true, true>(A, sa, B, sb, M, N, R, C, st, nullptr);
}

}  // namespace

hipError_t launch_gemm(const uint8_t* A, int fa, bool ta, const fp8_scale_t* sa, const uint8_t* B, int fb,
                       bool tb, const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R, void* C, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (fa == FP8_E4M3 && fb == FP8_E4M3) return launch_layouts<0, 0>(A, ta, sa, B, tb, sb, M, N, R, C, st);
  if (fa == FP8_E5M2 && fb == FP8_E4M3) return launch_layouts<1, 0>(A, ta, sa, B, tb, sb, M, N, R, C, st);
  if (fa == FP8_E4M3 && fb == FP8_E5M2) return launch_layouts<0, 1>(A, ta, sa, B, tb, sb, M, N, R, C, st);
  return launch_layouts<1, 1>(A, ta, sa, B, tb, sb, M, N, R, C, st);
}

bool gemm_pair_fused(const GemmDesc& g0, const GemmDesc& g1) {
  return g0.fa == FP8_E5M2 && g0.fb == FP8_E4M3 && !g0.ta && !g0.tb && g1.fa == FP8_E4M3 && g1.fb == FP8_E5M2 &&
         g1.ta && g1.tb;
}

hipError_t launch_gemm_pair(const GemmDesc& g0, const GemmDesc& g1, hipStream_t st) {
  const bool e0 = g0.M == 0 || g0.N == 0, e1 = g1.M == 0 || g1.N == 0;
  if (e0 || e1 || !gemm_pair_fused(g0, g1)) {
    hipError_t e = hipSuccess;
    if (!e0) e = launch_gemm(g0.A, g0.fa, g0.ta, g0.sa, g0.B, g0.fb, g0.tb, g0.sb, g0.M, g0.N, g0.R, g0.C, st);
    if (e == hipSuccess && !e1)
      e = launch_gemm(g1.A, g1.fa, g1.ta, g1.sa, g1.B, g1.fb, g1.tb, g1.sb, g1.M, g1.N, g1.R, g1.C, st);
    return e;
  }
  constexpr int E4 = FP8_E4M3, E5 = FP8_E5M2;
  const GemmParams p0 = make_params(g0.A, g0.sa, g0.B, g0.sb, g0.M, g0.N, g0.R, g0.C);
  const GemmParams p1 = make_params(g1.A, g1.sa, g1.B, g1.sb, g1.M, g1.N, g1.R, g1.C);
  const int blocks = p0.tiles_m * p0.tiles_n + p1.tiles_m * p1.tiles_n;
  hipLaunchKernelGGL((gemm_pair_kernel<E5, E4, false, false, E4, E5, true, true>), dim3(blocks), dim3(kThreads), 0,
                     st, p0, p1);
  return hipGetLastError();
}

TailSplit gemm_tail_split(int fa, int fb, int64_t M, int64_t N, int64_t R, int mode) {
  TailSplit ts{0, 0, 0};
  if (fa != FP8_E4M3 || fb != FP8_E4M3 || M <= 0 || N <= 0 || R < 512 || R % 256) return ts;
  if (mode == FP8_SPLIT_NEVER || (mode == FP8_SPLIT_AUTO && R < kSplitMinR)) return ts;
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  const int ncu = cu_count();
  const int64_t tail = tiles % ncu;
  if (tail == 0 || 2 * tail > ncu) return ts;  // whole waves, or a tail too wide to split into one wave
  ts.nfull = (int)(tiles - tail);
  ts.ntail = (int)tail;
  ts.bytes = (size_t)tail * 2 * 65536 * sizeof(float);
  return ts;
}

hipError_t launch_gemm_ws(const uint8_t* A, int fa, bool ta, const fp8_scale_t* sa, const uint8_t* B, int fb,
                          bool tb, const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R, void* C, int mode,
                          void* ws, size_t ws_bytes, hipStream_t st) {
  const TailSplit ts = gemm_tail_split(fa, fb, M, N, R, mode);
  if (ts.ntail == 0 || !ws || ws_bytes < ts.bytes)
    return launch_gemm(A, fa, ta, sa, B, fb, tb, sb, M, N, R, C, st);
  float* part = (float*)ws;
  if (!ta && !tb) return launch_tailsplit<false, false>(A, sa, B, sb, M, N, R, C, ts, part, st);
  if (!ta && tb) return launch_tailsplit<false, true>(A, sa, B, sb, M, N, R, C, ts, part, st);
  if (ta && !tb) return launch_tailsplit<true, false>(A, sa, B, sb, M, N, R, C, ts, part, st);
  return launch_tailsplit<true, true>(A, sa, B, sb, M, N, R, C, ts, part, st);
}

// Scratch memory of fp8_gemm_noalloc: the tail split's FP32 partials for
// up to kStaticTailTiles tiles (two 256 x 256 halves each), held in the
// code object's own device memory, so a call needs no workspace from the
// caller and allocates nothing. Each device that loads the library holds
// its own copy until the process ends. Host code never uses the array's
// name as an address: static_scratch() asks the runtime for this device's
// address once and keeps it.
constexpr size_t kStaticScratchBytes = (size_t)kStaticTailTiles * 2 * 65536 * sizeof(float);
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

hipError_t launch_gemm_wgrad_amax(const uint8_t* A, bool ta, const fp8_scale_t* sa, const uint8_t* B, bool tb,
                                  const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R, void* C,
                                  fp8_scale_t* s_out, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  constexpr int E4 = FP8_E4M3, E5 = FP8_E5M2;
  if (!ta && !tb) return launch_typed<E4, E5, true, false, false>(A, sa, B, sb, M, N, R, C, st, s_out);
  if (!ta && tb) return launch_typed<E4, E5, true, false, true>(A, sa, B, sb, M, N, R, C, st, s_out);
  if (ta && !tb) return launch_typed<E4, E5, true, true, false>(A, sa, B, sb, M, N, R, C, st, s_out);
  return launch_typed<E4, E5, true, true, true>(A, sa, B, sb, M, N, R, C, st, s_out);
}

}  // namespace fp8lin
