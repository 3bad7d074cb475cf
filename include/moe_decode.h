/*
 * moe_decode.h -- C ABI of the MI355X (gfx950) small-batch decode MoE FFN.
 *
 * One layer's FFN half at decode width M <= 48 token rows, on one GPU:
 *
 *   y    = RMSNorm(x) * norm_w, rounded to bf16                 (the FFN seam)
 *   x8   = MXFP8(y): E4M3 values, one E8M0 code per 32 columns
 *   s    = sigmoid(y . gate_w^T); picks = top-k of s + bias; w = s_pick / sum
 *   per picked expert e and for the shared expert:
 *     h  = x8 . W13[e]^T  (E4M3 x E4M3 with 32 x 32 E8M0 weight blocks)
 *     a8 = MXFP8(SiLU(h[:, :I]) * h[:, I:])
 *     ye = a8 . W2[e]^T
 *   out  = bf16(sum_j w_j ye_j + y_shared)
 *
 * Sources (three API-reference pages of one decode-layer implementation):
 *   "vllm.models.deepseek_v41.amd.mono.runner": DSV41MonoLayer.ffn (the FFN
 *     launch and its MoE tensors), DSV41MonoLayer.supports (1 <= M <= 48),
 *     DSV41MonoLayer.scratch (scratch allocated before any graph capture),
 *     MonoLayerWeights.check (tensor shapes and dtypes; 32 x 32 E8M0 blocks),
 *     _check_tensors (shape checks because loads are unbounded).
 *   "vllm.models.deepseek_v41.amd.mono.layer": run_ffn (norm, then the MoE
 *     and its output), store_normed (bf16 normed row), store_x8 (MXFP8).
 *   "vllm.models.deepseek_v41.amd.mono.attention.device": mx_code, mx_mul,
 *     fp8_pack4, mfma_scaled.
 *
 * Conventions for every entry point:
 *   - Pointers named d_* are device pointers on the device that was current
 *     when the plan was made; h_* are host pointers.
 *   - The library never allocates, frees or synchronises inside
 *     moe_decode_run: all device memory it needs is allocated by
 *     moe_decode_plan.  moe_decode_run enqueues its kernels on `stream` and
 *     returns; it may be captured into a HIP graph.
 *   - Return values: 0 on success, a negative MOE_DECODE_E* code otherwise;
 *     moe_decode_strerror() names it.  On an argument error nothing is
 *     enqueued.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_DECODE_OK 0
#define MOE_DECODE_EINVAL (-1)   /* a dimension, size, pointer or alignment is invalid */
#define MOE_DECODE_ENOMEM (-2)   /* device or host allocation failed */
#define MOE_DECODE_EHIP (-3)     /* a HIP runtime call failed (see moe_decode_last_hip_error) */
#define MOE_DECODE_ECAPTURE (-4) /* moe_decode_plan called while the stream is capturing */

/* Largest decode width the pages' runner supports (DSV41MonoLayer.supports). */
#define MOE_DECODE_MAX_TOKENS 48

/* Routed expert weight formats (the shared expert is always E4M3 with
 * 32 x 32 blocks). */
#define MOE_DECODE_ROUTED_E4M3 0  /* E4M3 [N, K] with E8M0 codes [N/32, K/32] */
#define MOE_DECODE_ROUTED_MXFP4 1 /* E2M1 pairs [N, K/2] (column 2i in the low
                                     nibble) with one E8M0 code per row and
                                     32 columns, in the blocked order
                                     [N/16][ceil(K/512)][16][16] (16-row tile,
                                     512-column segment, row, 32-column block):
                                     the pages' A8W4 routed experts
                                     (MonoLayerWeights.check, fp4x2) */

/* How runs are scheduled.  LAUNCHES: the short launches (seam, logits,
 * route, w13, SiLU * up, w2, combine; steps of up to 4 rows route inside
 * w13).  PERSISTENT: steps of at most 4 rows whose layer the persistent
 * launch covers run the seam, the router, w13, SiLU * up and w2 in one
 * launch of one block per CU, then the combine launch (the pages'
 * persistent MoE launch whose phases hand off through device counters:
 * [layer] run_ffn, build_mono_ffn; [device] atomic_add_dev); other steps run
 * the short launches.  The persistent launch cuts every active expert's
 * intermediate into one slice per XCD, and each XCD's blocks meet at a
 * barrier (a count in that XCD's L2) between w13, SiLU * up and w2, so
 * each hand-off stays in one XCD's L2.  It covers E4M3 routed experts whose I and Is are 2048 or 4096, with
 * the other conditions of the w13 launch that routes (below); the plan
 * checks that the device deals a launch's blocks to its XCDs round-robin
 * (from any first XCD), else every step runs the short launches.  It
 * assumes that all its blocks are resident at once; a wait past 100 ms sets
 * a status bit (moe_decode_status).  AUTO (the default): the schedule that
 * runs a step fastest on MI355X, today the short launches at every width.
 * Within one plan a token's output bits do not depend on the step's width.
 * Plans of the persistent schedule add w2 over 256-column segments where I
 * or Is is 2048 (its XCD slices), other plans over 512-column ones, so the
 * two can differ in the rounding of those sums. */
#define MOE_DECODE_SCHEDULE_AUTO 0
#define MOE_DECODE_SCHEDULE_LAUNCHES 1
#define MOE_DECODE_SCHEDULE_PERSISTENT 2

/* Layer dimensions, fixed when the plan is made.
 *   hidden        H, a multiple of 128 (the scaled MFMA's K step), <= 16384
 *   experts       E routed experts, 1..1024
 *   topk          k experts per token, 1..min(E, 32)
 *   inter         I, routed expert intermediate, a multiple of 128, <= 8192
 *   shared_inter  Is, shared expert intermediate, a multiple of 128, <= 8192
 *   max_tokens    largest m a run may pass, 1..48
 *   rms_eps       RMSNorm epsilon (added to mean(x^2) in double precision)
 *   routed_scale  factor applied to the renormalised routing weights
 *   routed_format MOE_DECODE_ROUTED_E4M3 or MOE_DECODE_ROUTED_MXFP4
 *   schedule      MOE_DECODE_SCHEDULE_AUTO, _LAUNCHES or _PERSISTENT */
typedef struct moe_decode_dims {
  int32_t hidden;
  int32_t experts;
  int32_t topk;
  int32_t inter;
  int32_t shared_inter;
  int32_t max_tokens;
  float rms_eps;
  float routed_scale;
  int32_t routed_format;
  int32_t schedule;
} moe_decode_dims;

typedef struct moe_decode_plan_s* moe_decode_handle;

/* Validates dims, allocates the plan's device scratch (laid out for
 * max_tokens rows) on the current device and zeroes it.  Must not be called
 * while a stream is being captured (DSV41MonoLayer.scratch raises in that
 * case; here: MOE_DECODE_ECAPTURE, checked on `stream`, which may be NULL for
 * the legacy stream).  On success *out owns the scratch until
 * moe_decode_destroy. */
int moe_decode_plan(const moe_decode_dims* dims, void* stream,
                    moe_decode_handle* out);

/* Device bytes the plan owns. */
size_t moe_decode_scratch_bytes(moe_decode_handle plan);

/* One decode step of m token rows, 1 <= m <= max_tokens (DSV41MonoLayer.ffn's
 * MoE pointers, with the norm weight, since the norm is on this path).
 *
 *   d_x       bf16 [m, H]            input rows (not modified)
 *   d_norm_w  bf16 [H]               RMSNorm weight
 *   d_gate_w  bf16 [E, H]            router weight
 *   d_bias    f32  [E]               expert-selection bias (e_score_correction_bias)
 *   d_w13     E4M3 [E, 2I, H]        rows [0, I) gate, [I, 2I) up
 *   d_w13_s   E8M0 [E, 2I/32, H/32]  one code per 32 x 32 block, row-major
 *   d_w2      E4M3 [E, H, I]
 *   d_w2_s    E8M0 [E, H/32, I/32]
 *             (MXFP4 routed experts: w13 [E, 2I, H/2] with codes
 *             [E, 2I/16, H/512, 16, 16], w2 [E, H, I/2] with codes
 *             [E, H/16, ceil(I/512), 16, 16], blocked as above)
 *   d_sgu     E4M3 [2Is, H]          shared expert gate/up
 *   d_sgu_s   E8M0 [2Is/32, H/32]
 *   d_sw2     E4M3 [H, Is]           shared expert down
 *   d_sw2_s   E8M0 [H/32, Is/32]
 *   d_out     bf16 [m, H]            written in full; must not alias any input
 *   stream    hipStream_t (NULL: the legacy stream)
 *
 * All tensors are dense row-major.  Every pointer must be non-NULL and 16-byte
 * aligned: the kernels' loads are unchecked against tensor bounds, so a tensor
 * smaller than its shape above is read past its end (the pages check shapes
 * on the host for the same reason, _check_tensors).  The caller keeps every
 * buffer alive until the enqueued work completes.  A plan serves one stream
 * at a time: two runs of one plan must not overlap (they share its scratch).
 * For m <= 4 (at most 64 pairs, E <= 256, H <= 8192, E at most twice the
 * CUs; the launches schedule) no seam launch runs: every block of the w13
 * launch normalises and quantises the rows into its LDS and sums the logits
 * of one or two experts; its first m blocks wait for those logits and route,
 * and the other blocks wait for the picks once the shared expert's units
 * are done.  The launch has one block per CU, so with all its blocks
 * resident every wait ends.  A wait that runs past 100 ms (another workload
 * holding CUs for that long) sets a bit of the status word
 * (moe_decode_status) and goes on.  The act launch clears the hand-off words for the next run; after a
 * run that returned an error between the w13 and act launches, the next run
 * launches the seam to clear them. */
int moe_decode_run(moe_decode_handle plan, int32_t m, const void* d_x,
                   const void* d_norm_w, const void* d_gate_w,
                   const float* d_bias, const void* d_w13,
                   const void* d_w13_s, const void* d_w2, const void* d_w2_s,
                   const void* d_sgu, const void* d_sgu_s, const void* d_sw2,
                   const void* d_sw2_s, void* d_out, void* stream);

/* The run for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): no plan, and no
 * allocation of any kind -- neither device nor host memory, nor a library
 * routine that allocates.  The same step as moe_decode_run with the same
 * kernels and output bits, on a plan-less scratch: one file-scope device
 * array of MOE_DECODE_NOALLOC_SCRATCH_BYTES per GPU the library runs on,
 * held until the process ends (its address is looked up once per device, on
 * the first call made with that device current).
 *   dims      as for moe_decode_plan (validated the same way); m <= max_tokens
 *   d_*       as for moe_decode_run
 *   d_status  u32 on the device: the bits moe_decode_status documents are
 *             ORed into it; the caller zeroes it and reads it after the
 *             step's work completes
 * The step's scratch is laid out for its m rows (not max_tokens'); a step
 * whose scratch would exceed the array returns MOE_DECODE_EINVAL (at
 * H = 5120, E = 256, top-8, I = Is = 2048 every m <= 48 fits).  Every call on
 * a GPU shares that GPU's array and leaves its contents there: two calls
 * whose work overlaps on one GPU (two streams, or two threads) race and give
 * wrong results; the caller serialises them.  Each step also launches the
 * seam kernel, which clears the array's hand-off words left by the previous
 * call.  Errors: EINVAL for bad dims, m, pointers or size, EHIP on a
 * runtime error (nothing is enqueued after an argument error). */
#define MOE_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_decode_run_noalloc(const moe_decode_dims* dims, int32_t m,
                           const void* d_x, const void* d_norm_w,
                           const void* d_gate_w, const float* d_bias,
                           const void* d_w13, const void* d_w13_s,
                           const void* d_w2, const void* d_w2_s,
                           const void* d_sgu, const void* d_sgu_s,
                           const void* d_sw2, const void* d_sw2_s,
                           void* d_out, uint32_t* d_status, void* stream);

/* Views of the last run's intermediates inside the plan's scratch (device
 * pointers, valid until the next run or destroy; read them after the run's
 * work completes).  Shapes use the last run's m; P = m * k pairs, R = P + m
 * rows (routed rows first, then one shared-expert row per token).
 *   NORMED    bf16 [m, H]       the RMSNorm output (store_normed)
 *   X8        u8   [m, H]       E4M3 of NORMED (store_x8)
 *   X8S       u8   [m, H/32]    E8M0 codes of X8
 *   LOGITS    f64  [m, E]       router logits
 *   TOPK_IDS  i32  [m, k]       picked experts in selection order
 *   TOPK_W    f32  [m, k]       routing weights of the picks
 *   COUNTS    i32  [E]          tokens per expert
 *   PAIR_ROW  i32  [m, k]       row of pair (t, j): pairs listed by expert
 *                               ascending, then token ascending
 *   ROW_TOK   i32  [R]          token of each row
 *   A8        u8   [R, Imax]    E4M3 SiLU*up intermediate (Imax = max(I, Is))
 *   A8S       u8   [R, Imax/32] its E8M0 codes
 *   STATUS    u32  [1]          the status word (see moe_decode_status) */
enum moe_decode_tap {
  MOE_DECODE_TAP_NORMED = 0,
  MOE_DECODE_TAP_X8 = 1,
  MOE_DECODE_TAP_X8S = 2,
  MOE_DECODE_TAP_LOGITS = 3,
  MOE_DECODE_TAP_TOPK_IDS = 4,
  MOE_DECODE_TAP_TOPK_W = 5,
  MOE_DECODE_TAP_COUNTS = 6,
  MOE_DECODE_TAP_PAIR_ROW = 7,
  MOE_DECODE_TAP_ROW_TOK = 8,
  MOE_DECODE_TAP_A8 = 9,
  MOE_DECODE_TAP_A8S = 10,
  MOE_DECODE_TAP_STATUS = 11
};
int moe_decode_inspect(moe_decode_handle plan, int32_t tap,
                       const void** d_ptr, size_t* bytes);

/* The plan's status word: 0 while every run since the last clear was valid.
 * A kernel that waits on other blocks of its launch (the hand-offs of the
 * pages' persistent launch through device-scope words, [device]
 * atomic_add_dev; [layer] run_ffn) gives up after 100 ms (or after
 * MOE_DECODE_WAIT_LIMIT_US microseconds when that environment variable is
 * set as a plan is made, or a no-alloc run starts: a low value makes the
 * waits give up at once, to check this path) and sets a bit; the
 * run's output is then not valid.  Bits: 1 a barrier of the persistent
 * launch (between its w13, SiLU * up and w2 phases); 2 a wait of a launch
 * that routes (m <= 4) for the logits or the picks; 4 blocks of the
 * persistent launch whose indices agree mod the XCD count ran on different
 * XCDs (their hand-offs then crossed XCDs).  The bits are sticky: no kernel
 * clears them, so a
 * check after many runs (a graph replayed many times) covers all of them.
 * moe_decode_status synchronises `stream`, copies the word to *h_status and,
 * when `clear` is nonzero, zeroes it.  Not during stream capture
 * (MOE_DECODE_ECAPTURE); EINVAL for a NULL plan or h_status; EHIP on a
 * runtime error. */
int moe_decode_status(moe_decode_handle plan, void* stream, uint32_t* h_status,
                      int32_t clear);

/* Per-kernel timing of runs: each kernel is launched with a start and a stop
 * HIP event that its dispatch itself records (hipExtLaunchKernelGGL), so an
 * interval is that kernel's execution on the run's stream.
 * moe_decode_timing(plan, 1) starts recording (and clears the totals), 0
 * stops.  While on, moe_decode_run must not be captured into a graph.
 * moe_decode_timing_read sums the elapsed milliseconds of kernel `kernel` (0
 * seam, 1 logits, 2 route, 3 w13, 4 act, 5 w2, 6 combine, 7 the persistent
 * launch) over the recorded
 * runs that launched it, and sets *runs to their number; it synchronises
 * with the recorded events.  (Steps of m <= 4 rows compute the logits inside
 * the seam launch and do not launch `logits`; with the launches schedule they
 * run the seam and the router inside w13 and launch neither.) */
int moe_decode_timing(moe_decode_handle plan, int32_t on);
int moe_decode_timing_read(moe_decode_handle plan, int32_t kernel,
                           double* total_ms, int32_t* runs);

/* Timeline of runs (the pages' timeline build: "layer" run_ffn's mark and
 * "device" stamp / memrealtime).  While on, thread 0 of every block of each
 * kernel stores the 100 MHz device clock (s_memrealtime) at fixed points:
 *   seam:  0 start, 1 squares summed, 2 logits (or rows) stored
 *   logits: 0 start, 1 end
 *   route: 0 start, 5 scores computed, 1 groups sorted, 6 lists merged,
 *          2 picks stored, 3 last block admitted, 4 plan written (3-4 only
 *          in the last block; 3 not with one token)
 *   w13, w2: 0 start, 3 + w: wave w of the block done, 1 end; w13 that
 *          routes also 2: its seam done (the route block's route points
 *          are stored as route's, block = token)
 *   persistent: 0 start, 2 seam done, 3 w13 phase done (wave 0), 4 SiLU *
 *          up phase done (wave 0), 5 and 6 the w2 phase done (the last
 *          even and the last odd wave to store), 1 end
 *   act, combine: 0 start, 1 end (thread 0's part)
 * Point 7 of every record holds where the block ran (XCC id << 32 | the
 * HW_ID register).  Blocks past the first 1024 of a launch are not recorded.
 * Unwritten points keep stale values.  moe_decode_timeline_read copies the
 * last run's records of kernel `kernel` (0 seam, 1 logits, 2 route, 3 w13,
 * 4 act, 5 w2, 6 combine, 7 persistent) as
 * u64 [blocks][8] into h_out (n entries available), sets *blocks, and
 * synchronises the device. */
int moe_decode_timeline(moe_decode_handle plan, int32_t on);
int moe_decode_timeline_read(moe_decode_handle plan, int32_t kernel,
                             uint64_t* h_out, size_t n, int32_t* blocks);

/* Frees the plan's scratch.  NULL is allowed. */
void moe_decode_destroy(moe_decode_handle plan);

/* Weight preparation (not part of a decode step): quantise a dense row-major
 * fp32 [rows, cols] matrix to E4M3 [rows, cols] with one E8M0 code per
 * 32 x 32 block ([rows/32, cols/32] row-major) -- the layout the expert
 * tensors above use (MonoLayerWeights.check: 32 x 32 E8M0 blocks).  Code per
 * block = clamp(ceil(log2(amax/448)) + 127, 0, 254) (mx_code); values are
 * rounded to nearest even after scaling by 2^(127 - code) (fp8_pack4).
 * rows and cols multiples of 32; pointers 16-byte aligned; `count` matrices
 * of that shape stored back to back are quantised in one call. */
int moe_decode_quantize_weight(const float* d_w, int32_t count, int32_t rows,
                               int32_t cols, void* d_q, void* d_scales,
                               void* stream);

/* Weight preparation for MXFP4 routed experts: quantise `count` back-to-back
 * fp32 [rows, cols] matrices to E2M1 pairs [rows, cols/2] (column 2i in the
 * low nibble) with one E8M0 code per row and 32 columns, stored in the
 * blocked order [rows/16][ceil(cols/512)][16][16] per matrix (the codes of a
 * 16-row, 512-column tile are one contiguous 256-byte block, row-major;
 * padding codes of a ragged last segment are 0).  Code = the smallest c in
 * [0, 254] with amax <= 6 * 2^(c-127); values rounded to nearest, ties to
 * the even mantissa bit, after scaling by 2^(127 - code).  rows a multiple
 * of 16, cols a multiple of 32; pointers 16-byte aligned. */
int moe_decode_quantize_weight_fp4(const float* d_w, int32_t count, int32_t rows,
                                   int32_t cols, void* d_q, void* d_scales,
                                   void* stream);

/* The seam upstream of the MoE ([layer] run_ffn: the attention's partials
 * summed and folded into the four-stream hyper-connection residual, whose
 * streams then give the FFN's input row; [runner] DSV41MonoLayer.ffn for
 * the shapes).  For each of m tokens (1 <= m <= 48) and column c < hidden:
 *   residual_out[t][i][c] = bf16(sum_j res[t][i][j] residual[t][j][c]
 *                                + post[t][i] part[t][c])       (i, j < 4)
 *   x[t][c] = bf16(sum_i pre[t][i] residual_out[t][i][c])
 * each sum in double precision in the order written, one rounding to nearest
 * even.  The pages give the tensors, not this arithmetic (the reading taken
 * here); the mixes of the FFN seam itself (its gate) are not computed: pre
 * is an input.
 *   d_part          bf16 [m, H]     attention output (TP-summed)
 *   d_residual      bf16 [m, 4, H]
 *   d_post          f32  [m, 4]     (the pages' [m, 4, 1])
 *   d_res           f32  [m, 4, 4]  res[t][i][j]: output stream i, input j
 *   d_pre           f32  [m, 4]
 *   d_residual_out  bf16 [m, 4, H]  may be d_residual itself (in place),
 *                                   else must not overlap it
 *   d_x             bf16 [m, H]     must not overlap any other argument
 * hidden a multiple of 128, <= 16384; pointers 16-byte aligned.  EINVAL on
 * bad arguments (nothing enqueued), EHIP on a failed launch. */
int moe_decode_hc_fold(int32_t m, int32_t hidden, const void* d_part,
                       const void* d_residual, const float* d_post,
                       const float* d_res, const float* d_pre,
                       void* d_residual_out, void* d_x, void* stream);

/* The attention seam's input quantisation ([layer] store_x8): the RMSNorm of
 * each row x [m, H] bf16 with weight d_norm_w bf16 [H] (the seam's chain:
 * sum of squares in double, r = 1/sqrt(ss/H + eps) rounded once to fp32,
 * two fp32 products; no bf16 rounding), then per 32 columns vLLM's ROCm
 * MXFP8 code of the amax ([device] mx_code: clamp(ceil(log2(amax / 448)) +
 * 127, 0, 254), amax floored at FLT_MIN), the values scaled by
 * 2^(127 - code), clamped to +-448 (clamp_fp8) and rounded to nearest even
 * E4M3.
 *   d_x8   u8 [m, H]     E4M3
 *   d_x8s  u8 [m, H/32]  E8M0 codes
 * 1 <= m <= 48, hidden a multiple of 128, <= 16384, rms_eps finite >= 0;
 * pointers 16-byte aligned.  EINVAL / EHIP as above. */
int moe_decode_attn_x8(int32_t m, int32_t hidden, const void* d_x,
                       const void* d_norm_w, float rms_eps, void* d_x8,
                       void* d_x8s, void* stream);

/* Measurement aid (not part of a decode step): the HBM read rate a plain
 * stream reaches on this device.  Reads the `bytes` bytes at d_buf once, in
 * 128-bit non-temporal loads (the width and cache policy of the expert
 * GEMMs' weight loads) from MOE_DECODE_PROBE_BLOCKS blocks of 256 threads,
 * sixteen loads in flight per thread, each block one contiguous range; time
 * it with events on `stream`.  Block b stores the XOR of the 32-bit words it
 * read at d_sink[b], so the XOR of all of d_sink is the XOR of every word of
 * the buffer.
 *   d_buf   16-byte aligned, bytes a multiple of 16 (>= 16)
 *   d_sink  u32 [MOE_DECODE_PROBE_BLOCKS], 4-byte aligned, fully overwritten
 * EINVAL on bad arguments (nothing enqueued), EHIP on a failed launch. */
#define MOE_DECODE_PROBE_BLOCKS 4096
int moe_decode_read_probe(const void* d_buf, size_t bytes, uint32_t* d_sink,
                          void* stream);

/* Text of an error code. */
const char* moe_decode_strerror(int code);
/* The last HIP error a plan (or, with NULL, the library) saw, as text. */
const char* moe_decode_last_hip_error(moe_decode_handle plan);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
