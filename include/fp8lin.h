/*
 * fp8lin.h - per-tensor dynamically scaled FP8 linear layer for MI355X (gfx950).
 *
 * C ABI of libfp8lin.so. Every entry point takes plain pointers and sizes and
 * enqueues HIP kernels on the stream it is given. The library never allocates
 * or frees memory, never synchronises the host with the device, never reads
 * device memory from the host, and keeps no pointer after returning; the
 * caller owns every buffer and must keep it alive until the stream work ends.
 * All device-side scale data stays on the device, so a whole forward/backward
 * step can be enqueued (or captured in a HIP graph) with no host round trip.
 * Calls that share a scaling record must run in stream order: two calls
 * on one record that overlap (different streams, no event between them)
 * race on its reduction words. Scalar arguments (margin, mu_log2, a fixed
 * bias, the Adam hyper-parameters and step) are kernel arguments, so a
 * captured graph replays them as captured.
 *
 * The method (sources cited by page title and section):
 *   [AMAX]  review of Perez, Zhang et al., "Training and inference of large
 *           language models using 8-bit floating point", section "Proposed
 *           method": per-tensor scaling biases from each tensor's max |x|
 *           (bullet 1); compute_bias = log2(format max / amax) with a
 *           configurable margin (bullet 2); scale before the FP8 cast and
 *           undo the scaling after the matmul (bullet 3); E4 format for
 *           weights and activations, E5 for gradients (bullet 4).
 *           The method also serves inference by post-training
 *           quantisation (bullet 5), and is compared with a fixed scaling
 *           bias, FP8-CSCALE (bullet 6; section "Main results", bullet 3:
 *           at 13B parameters a fixed bias converges only in [-1, 0]).
 *   [FP8LM] reading note on Peng et al., "FP8-LM: Training FP8 Large
 *           Language Models", section "Proposed method", O1, Eq. 3:
 *           gradients are multiplied by an auto-scaling factor mu, changed
 *           dynamically (the policy is not given; see fp8_wgrad_fp8).
 *
 * Readings where the pages are silent: OCP E4M3FN (max 448, no inf) and
 * E5M2 (max 57344); encode by round-to-nearest-even with saturation to
 * +-max (inf included), NaN -> 0x7F|sign; bias = floor(log2(max/amax)) -
 * margin + mu_log2 clamped to [-126, 126]; scale = 2^bias exactly; GEMM
 * outputs are bf16, rounded to nearest even from the FP32 accumulator.
 *
 * Errors: every function checks its arguments before enqueuing anything and
 * returns a status; it never aborts. Data-dependent conditions (a NaN in a
 * tensor, a zero tensor, a clamped bias) are reported in fp8_scale_t.flags
 * on the device, never as a status.
 *
 * Concurrency: calls that share an fp8_scale_t or an output buffer must be
 * ordered on one stream (or by events); otherwise they race.
 */
#ifndef FP8LIN_H
#define FP8LIN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8LIN_ABI_VERSION 13

typedef enum fp8_fmt {
  FP8_E4M3 = 0, /* OCP E4M3FN: weights and activations [AMAX bullet 4] */
  FP8_E5M2 = 1  /* OCP E5M2: gradients [AMAX bullet 4] */
} fp8_fmt;

typedef enum fp8_status {
  FP8_OK = 0,
  FP8_ERR_INVALID = 1,     /* null / misaligned pointer, negative size, bad enum, out-of-range int */
  FP8_ERR_UNSUPPORTED = 2, /* well-formed but outside what the kernels handle (e.g. a dim not a multiple of 16) */
  FP8_ERR_HIP = 3          /* a HIP launch or runtime call failed */
} fp8_status;

/* flags in fp8_scale_t */
#define FP8_FLAG_NONFINITE 1u /* the tensor holds a NaN or an inf: bias forced to 0 */
#define FP8_FLAG_ZERO 2u      /* amax == 0: bias forced to 0 */
#define FP8_FLAG_CLAMPED 4u   /* the bias rule left [-126, 126] and was clamped */

/*
 * Per-tensor scaling record. Lives in DEVICE memory, 64 bytes, 16-byte
 * aligned. The public fields are written by fp8_amax / fp8_scale /
 * fp8_amax_scale / fp8_quantize and read by fp8_cast and fp8_gemm_nt.
 *   amax      max |t| over the tensor (a bf16 value widened to fp32); NaN if
 *             the tensor holds a NaN, +inf if it holds an inf and no NaN.
 *   bias      the integer exponent bias b [AMAX bullet 2].
 *   scale     2^b: multiplies the tensor before the FP8 cast [AMAX bullet 3].
 *   scale_inv 2^-b: undoes the scale after the GEMM.
 *   flags     FP8_FLAG_* bits.
 * gen_max is the working word of the amax reductions (fp8_amax,
 * fp8_amax_scale, fp8_quantize, fp8_wgrad_fp8): (tag << 16) | bf16
 * magnitude bits, merged by atomic max. A call's tag is epoch + 1, and the
 * kernel that consumes the maximum (the cast, or the publish kernel of
 * fp8_amax) sets epoch to that tag, so every call outranks what earlier
 * calls left and the word is never cleared. Both words live on the device
 * and change only inside kernels, so a captured HIP graph replays
 * correctly (a host-side call counter would be frozen into the graph).
 * reduce_bits is the working word of the O2 Adam calls (fp32 magnitude
 * bits of a running max, cleared by the call that consumes it). All three
 * must be zero before the first call on the record (allocate zeroed memory
 * or call fp8_scale_reset once).
 */
typedef struct fp8_scale_t {
  float amax;
  int32_t bias;
  float scale;
  float scale_inv;
  uint32_t flags;
  uint32_t reduce_bits;   /* internal: running max of the |bf16| bit patterns */
  int32_t spec_bias;      /* internal: the bias fp8_quantize_spec's cast guessed */
  uint32_t sat_count;     /* elements saturated by the last fp8_wgrad_fp8 cast */
  uint64_t gen_max;       /* internal: tagged running max */
  uint64_t epoch;         /* internal: tag of the last maximum consumed */
  uint64_t reserved2[2];
} fp8_scale_t;

/* Human-readable name of a status. Never NULL. */
const char* fp8_status_str(fp8_status status);

/* FP8LIN_ABI_VERSION of the built library. */
int fp8_abi_version(void);

/*
 * Zero `count` scaling records (all fields) on `stream` with a kernel (no
 * hipMemset, so it may be captured in a graph). s_dev: device, 16-B aligned.
 */
fp8_status fp8_scale_reset(fp8_scale_t* s_dev, int64_t count, hipStream_t stream);

/*
 * a1 - amax [AMAX bullet 1]: max |x| over n bf16 values, one pass over HBM.
 *   x_bf16  device, n bf16 values, 16-B aligned (n may be 0: amax = 0).
 *   s_dev   device record; writes amax and flags (NONFINITE / ZERO), sets
 *           bias = 0, scale = scale_inv = 1 (call fp8_scale next).
 */
fp8_status fp8_amax(const void* x_bf16, int64_t n, fp8_scale_t* s_dev, hipStream_t stream);

/*
 * a2 - scale choice [AMAX bullet 2; FP8LM O1 Eq. 3], from s_dev->amax:
 *   bias = clamp(floor(log2(fmt_max / amax)) - margin + mu_log2, -126, 126)
 *   with fmt_max = 448 (E4M3) or 57344 (E5M2); amax = 0 or non-finite ->
 *   bias 0 plus a flag. Writes bias, scale, scale_inv, flags.
 *   margin, mu_log2: |value| <= 1024, else FP8_ERR_INVALID. mu = 2^mu_log2
 *   is the gradient auto-scaling factor (pass 0 for weights/activations).
 */
fp8_status fp8_scale(fp8_fmt fmt, int margin, int mu_log2, fp8_scale_t* s_dev, hipStream_t stream);

/* a1 + a2 fused: the reduction, then one publishing thread that writes
 * amax, bias, scale, scale_inv and flags (no separate fp8_scale call). */
fp8_status fp8_amax_scale(const void* x_bf16, int64_t n, fp8_fmt fmt, int margin, int mu_log2,
                          fp8_scale_t* s_dev, hipStream_t stream);

/*
 * The a2 rule [AMAX bullet 2: bias = log2(format max / amax) with a
 * configurable margin; FP8LM O1 Eq. 3: mu = 2^mu_log2 scales gradients] on
 * the host for one amax value (the same code the kernels run). Returns the
 * bias; *flags_out (nullable) receives FP8_FLAG_* bits. Out-of-range
 * margin/mu_log2 are clamped to +-1024. Pure host function: no device
 * memory, no stream, never fails.
 */
int32_t fp8_bias_host(float amax, fp8_fmt fmt, int margin, int mu_log2, uint32_t* flags_out);

/*
 * a1 + a2 + a3 fused (the hot path of fp8_linear_fwd / fp8_linear_bwd):
 * amax of x, the scale rule, and the cast (+ transpose), in two kernel
 * launches. The amax pass ends without any cross-block handshake; the cast
 * kernel derives the bias from the merged maximum itself and writes the
 * record's public fields, so the result equals fp8_amax_scale followed by
 * fp8_cast. Arguments as for those two calls (x [rows, cols] bf16, rows and
 * cols multiples of 16; out_rowwise / out_transposed nullable).
 */
fp8_status fp8_quantize(const void* x_bf16, int64_t rows, int64_t cols, fp8_fmt fmt, int margin,
                        int mu_log2, fp8_scale_t* s_dev, uint8_t* out_rowwise, uint8_t* out_transposed,
                        hipStream_t stream);

/*
 * a1 + a2 + a3 [AMAX bullets 1-4] in one pass over x plus a check: the
 * cast uses the bias the record holds from its previous quantisation (a
 * guess) while the same pass takes max |x|; a second kernel derives the
 * bias from that max by the rule of fp8_quantize and, only where it
 * differs from the guess, recasts x with it. The record and every byte of
 * out_rowwise equal fp8_quantize's (the guess only decides how much work
 * is done): 2 B read + 1 B written per element when the bias repeats, 4 +
 * 2 when it changes (a fresh record holds bias 0). Arguments as for
 * fp8_quantize, row-major output only (out_rowwise required). The record
 * must have been zeroed once; its spec_bias word is internal.
 */
fp8_status fp8_quantize_spec(const void* x_bf16, int64_t rows, int64_t cols, fp8_fmt fmt, int margin,
                             int mu_log2, fp8_scale_t* s_dev, uint8_t* out_rowwise, hipStream_t stream);

/* Most tensors one fp8_quantize_batch call takes. */
#define FP8_QUANTIZE_BATCH_MAX 4

/* The arguments of one fp8_quantize call. */
typedef struct fp8_quantize_args {
  const void* x;             /* bf16 [rows, cols], device */
  int64_t rows, cols;
  fp8_fmt fmt;
  int margin, mu_log2;
  fp8_scale_t* s;            /* the tensor's own record (device) */
  uint8_t* out_rowwise;      /* nullable */
  uint8_t* out_transposed;   /* nullable */
} fp8_quantize_args;

/*
 * a1 + a2 + a3 [AMAX bullets 1-4; FP8LM O1 Eq. 3 for mu] for up to
 * FP8_QUANTIZE_BATCH_MAX tensors in two kernel launches (one amax pass
 * over all of them, then all their casts), each
 * tensor with its own per-tensor scale exactly as fp8_quantize computes it
 * (same record fields, bit-identical FP8 bytes). For tensors that are ready
 * together, such as a linear's X and W before its forward GEMM: one launch
 * pair instead of one per tensor, whose grids share the chip in
 * proportion to the tensors' sizes.
 *   tensors: host array of count argument sets, read during the call only;
 *   1 <= count <= FP8_QUANTIZE_BATCH_MAX, else FP8_ERR_INVALID. Each set
 *   is checked as fp8_quantize checks its arguments (the first failing
 *   status is returned, nothing enqueued). The records must be distinct
 *   (FP8_ERR_INVALID otherwise); no output may overlap another tensor's
 *   input, output or record.
 */
fp8_status fp8_quantize_batch(const fp8_quantize_args* tensors, int count, hipStream_t stream);

/*
 * FP8-CSCALE fixed scaling [AMAX "Proposed method" bullet 6, "Main results"
 * bullet 3]: set a record to a constant bias instead of deriving it from the
 * tensor's amax. Writes amax = 0, bias, scale = 2^bias, scale_inv = 2^-bias,
 * flags = 0 (the internal words are left as they are), so that fp8_cast and
 * fp8_gemm_nt use the record exactly as they use an amax-derived one.
 *   s_dev  device record, 16-B aligned.
 *   bias   in [-126, 126], else FP8_ERR_INVALID.
 */
fp8_status fp8_scale_fixed(fp8_scale_t* s_dev, int32_t bias, hipStream_t stream);

/*
 * a3 - cast (+ transpose) [AMAX bullets 3-4]: q = enc_fmt(x * 2^bias) with
 * round-to-nearest-even, saturation to +-max, subnormals kept, NaN ->
 * 0x7F|sign (whatever the record's flags say, e.g. a fixed-bias record);
 * bias from s_dev (device).
 *   x_bf16          device, [rows, cols] row-major bf16, 16-B aligned.
 *   out_rowwise     device, [rows, cols] u8, or NULL to skip.
 *   out_transposed  device, [cols, rows] u8, or NULL to skip.
 *   rows, cols      >= 0 and multiples of 16 (else FP8_ERR_UNSUPPORTED).
 */
fp8_status fp8_cast(const void* x_bf16, int64_t rows, int64_t cols, fp8_fmt fmt,
                    const fp8_scale_t* s_dev, uint8_t* out_rowwise, uint8_t* out_transposed,
                    hipStream_t stream);

/*
 * a4-a6 - FP8 GEMM, NT form, FP32 accumulation on FP8 MFMA, dequantising
 * bf16 epilogue [AMAX bullet 3]:
 *   C[i, j] = bf16_rne( 2^-(sa.bias + sb.bias) * sum_r A[i, r] * B[j, r] )
 *   A   device, [M, R] u8 codes of format fa, row-major (r contiguous).
 *   B   device, [N, R] u8 codes of format fb, row-major (r contiguous).
 *   C   device, [M, N] bf16 row-major (overwritten).
 *   sa, sb  device scaling records of A and B.
 *   M, N, R >= 0 and multiples of 16, and A and B each below 4 GiB
 *   (M*R, N*R < 2^32), else FP8_ERR_UNSUPPORTED; R = 0 gives C = 0.
 *   Forward:  Y  = gemm(A = x8 [M,K],  B = w8t [N,K])
 *   Dgrad:    dX = gemm(A = dy8 [M,N], B = w8 [K,N])      (E5M2 x E4M3)
 *   Wgrad:    dW = gemm(A = x8t [K,M], B = dy8t [N,M])    (E4M3 x E5M2)
 * All pointers 16-B aligned.
 */
fp8_status fp8_gemm_nt(const uint8_t* A, fp8_fmt fa, const fp8_scale_t* sa, const uint8_t* B,
                       fp8_fmt fb, const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R,
                       void* C_bf16, hipStream_t stream);

/* How a GEMM operand is stored. */
typedef enum {
  FP8_OPERAND_ROWS = 0, /* one row per output index, reduction contiguous: A [M,R], B [N,R] */
  FP8_OPERAND_COLS = 1  /* reduction-major: A [R,M], B [R,N] (the row-major FP8 copy of the
                           tensor that was cast, read transposed) */
} fp8_layout;

/*
 * a4-a6 - the same GEMM with either operand in either layout (same
 * arguments, rules and result as fp8_gemm_nt, which is la = lb = ROWS):
 *   C[i, j] = bf16_rne( 2^-(sa.bias + sb.bias) * sum_r A(i, r) * B(j, r) )
 * with A(i, r) = A[i, r] (ROWS) or A[r, i] (COLS), B likewise. With COLS the
 * transposed FP8 copies are not needed:
 *   Forward:  Y  = gemm(A = x8 [M,K] ROWS,  B = w8 [K,N] COLS)
 *   Dgrad:    dX = gemm(A = dy8 [M,N] ROWS, B = w8 [K,N] ROWS)
 *   Wgrad:    dW = gemm(A = x8 [M,K] COLS,  B = dy8 [M,N] COLS)
 * la, lb outside fp8_layout -> FP8_ERR_INVALID.
 */
fp8_status fp8_gemm(const uint8_t* A, fp8_fmt fa, fp8_layout la, const fp8_scale_t* sa, const uint8_t* B,
                    fp8_fmt fb, fp8_layout lb, const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R,
                    void* C_bf16, hipStream_t stream);

/* When fp8_gemm_ws splits the last wave of a GEMM. */
typedef enum {
  FP8_SPLIT_AUTO = 0,  /* when it pays: the conditions below and R >= 16384 */
  FP8_SPLIT_NEVER = 1,
  FP8_SPLIT_TAIL = 2   /* whenever the conditions below hold (R >= 512) */
} fp8_split;

/*
 * Workspace bytes fp8_gemm_ws [AMAX bullet 3] uses for this GEMM on the
 * current device with this split mode: 0 when it would not split. Only E4M3 x E4M3 GEMMs
 * (the forward) with R a multiple of 256 split: when the output tiles
 * (256 x 256) leave a last wave at most half full on the device's CUs,
 * each tile of that wave is computed as two reduction halves (FP32
 * partial sums, 512 KiB per tile) that a second kernel adds, so the last
 * wave runs twice as many blocks of half the length. The fixup launch and
 * the partials' traffic outweigh the saving for short reductions
 * (measured on the GPT-13B/175B-style forward GEMMs: R = 5120-12288
 * 4-9 % slower, R = 20480 3 % and R = 49152 12 % faster), hence the
 * AUTO threshold. Negative sizes give 0.
 */
size_t fp8_gemm_workspace_bytes(fp8_fmt fa, fp8_fmt fb, int64_t M, int64_t N, int64_t R, fp8_split split);

/*
 * a4 - fp8_gemm with a caller workspace [AMAX bullet 3: the matmul on the
 * scaled FP8 operands, the scaling undone after it] (same arguments,
 * checks and result bound): when fp8_gemm_workspace_bytes (same split mode) is nonzero and
 * workspace_bytes covers it, the last partial wave's tiles are split as
 * described there (two launches: the GEMM and the fixup), else this is
 * fp8_gemm. split outside fp8_split -> FP8_ERR_INVALID. A split
 * tile's sum is half0 + half1 in FP32, so it may differ from fp8_gemm's
 * result by accumulation order (inside the GEMM tolerance); the result is
 * deterministic. workspace: device, 16-B aligned, or NULL (no split); not
 * read before it is written; concurrent calls must not share it.
 */
fp8_status fp8_gemm_ws(const uint8_t* A, fp8_fmt fa, fp8_layout la, const fp8_scale_t* sa, const uint8_t* B,
                       fp8_fmt fb, fp8_layout lb, const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R,
                       void* C_bf16, fp8_split split, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Bytes of the device scratch fp8_gemm_noalloc uses (the tail split's FP32
 * partials of at most 128 tiles: 64 MiB, held per device from library load
 * to process end). */
#define FP8_NOALLOC_SCRATCH_BYTES ((size_t)128 * 2 * 65536 * 4)

/*
 * fp8_gemm_ws without a caller workspace, for callers that cannot allocate
 * device memory or bring a workspace: code being captured into a HIP graph,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * checks and result as fp8_gemm_ws (same kernels: bit-identical output),
 * with the tail split's partials in a scratch array the library's code
 * object holds on each device (FP8_NOALLOC_SCRATCH_BYTES). The call
 * allocates nothing; its first call on a device looks up that device's
 * scratch address (the current device must be the stream's). A split
 * that would need more than the scratch holds -> FP8_ERR_UNSUPPORTED
 * (nothing enqueued; with at most 256 CUs every split fits). Every call
 * on a device shares that device's scratch: calls that may overlap on one
 * GPU (different streams, no event between them) race and must be
 * serialised by the caller. The scratch is written before it is read
 * within a call, so nothing needs clearing between calls.
 */
fp8_status fp8_gemm_noalloc(const uint8_t* A, fp8_fmt fa, fp8_layout la, const fp8_scale_t* sa, const uint8_t* B,
                            fp8_fmt fb, fp8_layout lb, const fp8_scale_t* sb, int64_t M, int64_t N, int64_t R,
                            void* C_bf16, fp8_split split, hipStream_t stream);

/* The arguments of one fp8_gemm call. */
typedef struct fp8_gemm_args {
  const uint8_t* A;
  fp8_fmt fa;
  fp8_layout la;
  const fp8_scale_t* sa;
  const uint8_t* B;
  fp8_fmt fb;
  fp8_layout lb;
  const fp8_scale_t* sb;
  int64_t M, N, R;
  void* C;
} fp8_gemm_args;

/*
 * a5 + a6 - two GEMMs enqueued together [AMAX bullets 3-4: the backward
 * matmuls on E5 gradients and E4 weights / activations], each computed
 * exactly as fp8_gemm computes it with the same arguments (same checks and statuses,
 * bit-identical results). When the pair is a linear's backward - first the
 * dgrad (A E5M2 ROWS, B E4M3 ROWS), then the wgrad (A E4M3 COLS, B E5M2
 * COLS) - both run in one kernel launch: the first GEMM's output tiles are
 * dispatched first and the second's fill its tail, which saves one
 * launch's ramp-up and drain. Any other pair is launched as two GEMMs in
 * order.
 *   first, second: host pointers to the argument sets, read during the
 *   call only. Both are validated before anything is enqueued (the first
 *   failing status is returned). The two GEMMs may run concurrently: the
 *   output of either must not overlap the other's inputs or output.
 */
fp8_status fp8_gemm_pair(const fp8_gemm_args* first, const fp8_gemm_args* second, hipStream_t stream);

/*
 * Workspace of one FP8 linear: device pointers owned by the caller.
 *   x8 [M,K], w8 [K,N], dy8 [M,N] (u8, row-major FP8 copies): required.
 *   x8t [K,M], w8t [N,K], dy8t [N,M] (transposed copies): optional, NULL
 *   to skip. The GEMMs read only the row-major copies (reduction-major
 *   where needed, see fp8_gemm); a transposed copy is written when its
 *   pointer is set, for callers that want it.
 *   sx, sw, sdy: zero-initialised scaling records (see fp8_scale_t).
 *   scratch, scratch_bytes: optional workspace of the forward GEMM
 *   (16-B aligned, or NULL; fp8_linear_scratch_bytes tells the size).
 * The forward fills x8, w8, sx, sw (and x8t, w8t if set); the backward
 * reads them and fills dy8, sdy (and dy8t if set).
 */
typedef struct fp8_linear_ws {
  uint8_t* x8;
  uint8_t* x8t;
  uint8_t* w8;
  uint8_t* w8t;
  uint8_t* dy8;
  uint8_t* dy8t;
  fp8_scale_t* sx;
  fp8_scale_t* sw;
  fp8_scale_t* sdy;
  void* scratch;          /* forward GEMM workspace (fp8_gemm_ws), or NULL */
  size_t scratch_bytes;
} fp8_linear_ws;

/* Scratch bytes that let fp8_linear_fwd split its GEMM's last wave
 * (fp8_gemm_workspace_bytes with FP8_SPLIT_AUTO) [AMAX bullet 3: the
 * matmul on the scaled FP8 operands, whose FP32 partial sums the split
 * keeps]; 0 when it would not. Negative sizes give 0. Host function, no
 * device access. */
size_t fp8_linear_scratch_bytes(int64_t M, int64_t K, int64_t N);

/*
 * Forward of one linear, Y = X W [AMAX "Proposed method" bullets 1-4:
 * per-tensor amax of X and W, bias = log2(max / amax) - margin, scale and
 * cast to E4M3, FP8 matmul, scaling undone after it; FP8LM O1 Eq. 3 for
 * the bias rule's form]: fp8_quantize of X and W (E4M3), then the forward
 * GEMM gemm(x8 ROWS, w8 COLS).
 *   X [M,K] bf16, W [K,N] bf16 (in x out), Y [M,N] bf16; device, 16-B aligned.
 *   M, K, N multiples of 16, every FP8 operand below 4 GiB. ws: host struct
 *   of device pointers (above), read during the call only; the buffers it
 *   names are the caller's and are written on the stream.
 *   margin: |margin| <= 1024. Errors: FP8_ERR_INVALID (null / misaligned
 *   pointer, negative size, bad margin, ws->sx == ws->sw),
 *   FP8_ERR_UNSUPPORTED (a size not a multiple of 16 or too large),
 *   FP8_ERR_HIP (launch failure); nothing is enqueued on an argument error.
 */
fp8_status fp8_linear_fwd(const void* X, const void* W, int64_t M, int64_t K, int64_t N, int margin,
                          const fp8_linear_ws* ws, void* Y, hipStream_t stream);
/* (X and W are quantised together, as one fp8_quantize_batch: ws->sx and
 * ws->sw must be distinct records, else FP8_ERR_INVALID.) */

/*
 * Backward of one linear [AMAX "Proposed method" bullets 1-4: amax of dY,
 * its bias with the margin, the E5 format for gradients, FP8 matmuls with
 * the scaling undone after them; FP8LM O1 Eq. 3: the gradient's bias also
 * takes log2 mu]: fp8_quantize of dY (E5M2, with mu = 2^mu_log2),
 * then dX = dY W^T = gemm(dy8 ROWS, w8 ROWS) and dW = X^T dY =
 * gemm(x8 COLS, dy8 COLS) from the FP8 copies the forward left in ws
 * (when both are asked for, as one fp8_gemm_pair launch).
 *   dY [M,N] bf16; dX [M,K] bf16 or NULL to skip; dW [K,N] bf16 or NULL to skip.
 *   margin, mu_log2: |value| <= 1024. ws->sdy must differ from ws->sx and
 *   ws->sw (FP8_ERR_INVALID otherwise: dY's quantise rewrites its record).
 *   Other errors as for fp8_linear_fwd.
 */
fp8_status fp8_linear_bwd(const void* dY, int64_t M, int64_t K, int64_t N, int margin, int mu_log2,
                          const fp8_linear_ws* ws, void* dX, void* dW, hipStream_t stream);

/*
 * FP8 weight gradient [FP8LM "Proposed method" O1: FP8 gradients with the
 * auto-scaling factor mu, g' = mu * g (Eq. 3); AMAX bullet 4: E5 for
 * gradients]: dW = X^T dY (the a6 GEMM) whose epilogue also takes max |dW|
 * over the bf16 values it writes, then dW cast to E5M2 with the bias from
 * that amax, the margin and mu = 2^mu_log2. The result equals the wgrad
 * GEMM followed by fp8_quantize(dW, E5M2, margin, mu_log2), without reading
 * dW again for its amax. s_dw->sat_count is set to the number of elements
 * whose scaled magnitude exceeded the E5M2 max (clipped to it; inf counts,
 * NaN does not): the signal a mu auto-scaling policy needs.
 *   x8 (E4M3, record sx) and dy8 (E5M2, record sdy), each in either
 *   layout, as operands A and B of fp8_gemm: lx = ROWS for X^T [K,M],
 *   COLS for the row-major X [M,K]; ldy = ROWS for dY^T [N,M], COLS for
 *   dY [M,N]. A layout outside fp8_layout -> FP8_ERR_INVALID.
 *   dW_bf16 [K,N] bf16: written (and read back by the cast).
 *   dw8 [K,N] u8 E5M2: written. dw8t [N,K] u8: written, or NULL to skip.
 *   s_dw: dW's record (written; zero its internal words once, as for any
 *   record). K, N, M multiples of 16, operands below 4 GiB; device
 *   pointers 16-B aligned.
 */
fp8_status fp8_wgrad_fp8(const uint8_t* x8, fp8_layout lx, const fp8_scale_t* sx, const uint8_t* dy8,
                         fp8_layout ldy, const fp8_scale_t* sdy, int64_t K, int64_t N, int64_t M, int margin,
                         int mu_log2, void* dW_bf16, fp8_scale_t* s_dw, uint8_t* dw8, uint8_t* dw8t,
                         hipStream_t stream);

/*
 * O2 optimizer state [FP8LM "Proposed method", O2: precision-decoupled Adam,
 * first moment FP8, second moment FP16, master weights FP16 with tensor
 * scaling, 6 bytes per parameter with the FP8 gradient]. Readings where the
 * page is silent: the first moment is E4M3 with a per-tensor record (as any
 * FP8 tensor here); the FP16 second moment and master weights each carry a
 * per-tensor power-of-two scale in a record (value = fp16 * scale_inv),
 * chosen as for the FP8 path with the FP16 max 65504; the update is AdamW
 * with bias correction in fp32; every new scale is taken just in time from
 * the new tensor's max |value|.
 *
 * fp8_adam_init_master: master weights from bf16 weights: w16 [n] FP16 and
 * its record s_w (amax rule with max 65504). The moments start as zero
 * bytes with zeroed records (they decode as 0).
 *
 * fp8_adam_step: one step on n parameters, in place:
 *   g  = dec_E5M2(g8) * s_g.scale_inv                      (e.g. fp8_wgrad_fp8)
 *   m1 = beta1 m1 + (1 - beta1) g;  m2 = beta2 m2 + (1 - beta2) g^2
 *   w  = w - lr ((m1 / (1 - beta1^step)) / (sqrt(m2 / (1 - beta2^step)) + eps) + weight_decay w)
 * then m1 re-encoded in E4M3 and m2, w in FP16 with new per-tensor scales
 * (records rewritten), and, if w_bf16 is not NULL, the new weights rounded
 * to bf16 there (the next forward's W). Three kernel launches; a record's
 * reduce_bits must be zero before the first call (fp8_scale_reset).
 *   n: multiple of 16; g8, m1 [n] u8; m2, w16 [n] fp16 bits; w_bf16 [n] bf16
 *   or NULL; all 16-B aligned device pointers. lr, eps, weight_decay finite
 *   with eps > 0 and weight_decay >= 0; 0 <= beta < 1; step >= 1;
 *   else FP8_ERR_INVALID.
 */
fp8_status fp8_adam_init_master(int64_t n, const void* w_bf16, uint16_t* w16, fp8_scale_t* s_w, hipStream_t stream);
fp8_status fp8_adam_step(int64_t n, const uint8_t* g8, const fp8_scale_t* s_g, uint8_t* m1, fp8_scale_t* s_m1,
                         uint16_t* m2, fp8_scale_t* s_m2, uint16_t* w16, fp8_scale_t* s_w, void* w_bf16, float lr,
                         float beta1, float beta2, float eps, float weight_decay, int32_t step, hipStream_t stream);

/*
 * fp8_adam_step_spec: the step of fp8_adam_step [FP8LM "Proposed method",
 * O2, as above] in one pass over the state in the common case, out of
 * place: reads g8, m1, m2, w16 and writes the new state to m1_out, m2_out,
 * w16_out (and the bf16 weights to w_bf16 if not NULL), encoded with the
 * scales the records hold now while the new maxima are taken; a second
 * kernel derives the new scales and, only where one differs from its
 * record's, recomputes every element from the untouched inputs with the
 * new scales. The records are then rewritten as by fp8_adam_step, and the
 * outputs and records equal fp8_adam_step's on the same inputs bit for bit.
 * HBM traffic 13 bytes per parameter (6 read, 7 written) when no scale
 * changes, 24 when one does.
 *   Arguments as fp8_adam_step; m1_out [n] u8, m2_out and w16_out [n] fp16
 *   bits, 16-B aligned, none overlapping an input or another output
 *   (else FP8_ERR_INVALID). missed: NULL or a device uint32, 4-B aligned,
 *   set to a bit mask of the records whose bias changed (bit 0 m1, bit 1
 *   m2, bit 2 w), i.e. the steps that took the second pass.
 */
fp8_status fp8_adam_step_spec(int64_t n, const uint8_t* g8, const fp8_scale_t* s_g, const uint8_t* m1,
                              const uint16_t* m2, const uint16_t* w16, uint8_t* m1_out, uint16_t* m2_out,
                              uint16_t* w16_out, fp8_scale_t* s_m1, fp8_scale_t* s_m2, fp8_scale_t* s_w,
                              void* w_bf16, uint32_t* missed, float lr, float beta1, float beta2, float eps,
                              float weight_decay, int32_t step, hipStream_t stream);

/* How fp8_linear_fwd_cached scales X. */
typedef enum fp8_scaling {
  FP8_SCALING_AMAX = 0,  /* just in time from amax(X) and the margin (FP8-AMAX) */
  FP8_SCALING_FIXED = 1  /* the bias already in sx, e.g. from fp8_scale_fixed (FP8-CSCALE) */
} fp8_scaling;

/*
 * FP8 inference forward with a weight cast once, as in post-training
 * quantisation [AMAX "Proposed method" bullet 5]: Y = X W from a prepared
 * FP8 weight w8 (E4M3, e.g. fp8_amax_scale + fp8_cast, or fp8_scale_fixed
 * + fp8_cast) and its record sw. lw = FP8_OPERAND_COLS: w8 is the row-major
 * copy of W [K,N] (the layout the training forward reads, and the faster
 * one: read reduction-major); FP8_OPERAND_ROWS: w8 is W's transposed copy
 * [N,K]; another value -> FP8_ERR_INVALID. Per call only X is
 * quantised: with FP8_SCALING_AMAX, amax + bias (margin) + the row-wise cast
 * into x8 with its record written to sx (as fp8_quantize with no transposed
 * output); with FP8_SCALING_FIXED, the row-wise cast with the bias sx holds.
 * Then the forward GEMM. Bit-identical to fp8_linear_fwd's Y (in either
 * layout) when w8 and sw are what fp8_linear_fwd would produce from W.
 *   X [M,K] bf16, Y [M,N] bf16, w8 u8, x8 [M,K] u8; device, 16-B
 *   aligned. M, K, N multiples of 16, x8 and w8 below 4 GiB.
 *   sw: read only. sx: written (AMAX) or read (FIXED); sx == sw ->
 *   FP8_ERR_INVALID. NaNs in X become NaN codes in either mode.
 */
fp8_status fp8_linear_fwd_cached(const void* X, int64_t M, int64_t K, int64_t N, int margin,
                                 fp8_scaling x_scaling, const uint8_t* w8, fp8_layout lw, const fp8_scale_t* sw,
                                 uint8_t* x8, fp8_scale_t* sx, void* Y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8LIN_H */
