/*
 * moe_oracle.h -- the CPU oracle of the small-batch decode MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the checker, not the product:
 * only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg may load or call it.  It shares no code, header, table or constant with
 * the HIP path, and it never reads anything the HIP path produced.
 *
 * Plain, slow, single-threaded C.  Every floating-point step is carried out
 * in double precision unless the pages fix the precision; the only roundings
 * are the ones the method itself defines (bf16 rows, fp32 norm scale, fp32
 * SiLU*up, E4M3 codes, the bf16 output).
 *
 * The pages are three API-reference pages of one decode-layer implementation:
 *   [layer]  "vllm.models.deepseek_v41.amd.mono.layer"
 *   [runner] "vllm.models.deepseek_v41.amd.mono.runner"
 *   [device] "vllm.models.deepseek_v41.amd.mono.attention.device"
 * Each function below names the page and the section it follows.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layer dimensions (the pages' MonoLayerWeights.check shapes, with the
 * expert count, top-k and intermediates as parameters). */
/* Routed expert weight formats: E4M3 with one E8M0 code per 32 x 32 block,
 * or MXFP4 (E2M1, two per byte) with one code per row and 32 columns. */
#define ORC_FMT_E4M3 0
#define ORC_FMT_MXFP4 1

typedef struct orc_dims {
  int32_t hidden;        /* H */
  int32_t experts;       /* E routed experts */
  int32_t topk;          /* k */
  int32_t inter;         /* I, routed expert intermediate */
  int32_t shared_inter;  /* Is, shared expert intermediate */
  float rms_eps;         /* RMSNorm epsilon */
  float routed_scale;    /* factor on the renormalised routing weights */
  int32_t routed_format; /* ORC_FMT_E4M3 or ORC_FMT_MXFP4 (the shared expert is E4M3) */
} orc_dims;

/* ---- number formats ---------------------------------------------------- */

/* bf16 bit pattern -> its exact value. */
double orc_bf16_value(uint16_t b);
/* The bf16 nearest to v, ties to even (one rounding from double). */
uint16_t orc_bf16_rne(double v);
/* E4M3 (float8_e4m3fn, max 448, 0x7F/0xFF NaN) byte -> exact value; NaN for
 * the two NaN codes.  [runner] MonoLayerWeights (e4m3 tensors). */
double orc_e4m3_value(uint8_t b);
/* The E4M3 byte nearest to v, ties to the even code; |v| is clamped to 448
 * first; the sign bit follows v's sign (negative values that round to zero
 * give 0x80).  [device] fp8_pack4 (round to nearest even). */
uint8_t orc_e4m3_rne(double v);
/* E8M0 scale code of a 32-group with largest magnitude amax: the smallest
 * integer c in [0, 254] with amax <= 448 * 2^(c-127), i.e.
 * clamp(ceil(log2(amax/448)) + 127, 0, 254) with every all-zero or tiny group
 * at 0.  [device] mx_code. */
int32_t orc_mx_code(double amax);

/* E2M1 (float4_e2m1fn) nibble -> exact value.  [runner] MonoLayerWeights
 * (the routed experts' fp4x2 tensors). */
double orc_e2m1_value(uint8_t nibble);
/* The E2M1 nibble nearest to v, ties to the even (zero) mantissa bit; |v|
 * saturates at 6; the sign bit follows v's sign. */
uint8_t orc_e2m1_rne(double v);
/* E8M0 code of a 32-value FP4 block: the smallest c in [0, 254] with
 * amax <= 6 * 2^(c-127). */
int32_t orc_fp4_code(double amax);

/* Element-wise loops over the scalar functions above (for tests that
 * sweep many inputs). */
void orc_e2m1_rne_array(int64_t n, const double* v, uint8_t* out);
void orc_e4m3_rne_array(int64_t n, const double* v, uint8_t* out);
void orc_mx_code_array(int64_t n, const double* amax, int32_t* out);
void orc_bf16_rne_array(int64_t n, const double* v, uint16_t* out);

/* ---- quantisers --------------------------------------------------------- */

/* MXFP8 of one row of n values (n % 32 == 0): per 32 contiguous values,
 * code = mx_code(amax), q = E4M3(v * 2^(127-code)).  [layer] store_x8. */
void orc_mx_quant_row(int32_t n, const double* v, uint8_t* q, uint8_t* codes);
/* MXFP8 of a [rows, cols] fp32 weight in 32 x 32 blocks; scales row-major
 * [rows/32, cols/32].  [runner] MonoLayerWeights.check / AttnWeights.check. */
void orc_quant_weight(int32_t rows, int32_t cols, const float* w, uint8_t* q,
                      uint8_t* scales);
/* Position of the code of row r, 32-column block b of an MXFP4 [rows, cols]
 * matrix in its blocked code array [rows/16][ceil(cols/512)][16][16]. */
size_t orc_fp4_code_index(int32_t cols, int32_t r, int32_t b);
/* MXFP4 of a [rows, cols] fp32 weight (rows % 16 == 0): one code per row and
 * 32 columns (orc_fp4_code of their amax) in the blocked order above, padding
 * codes 0; elements E2M1 two per byte, column 2i in the low nibble.
 * [runner] MonoLayerWeights.check (w13, w2 fp4x2). */
void orc_quant_weight_fp4(int32_t rows, int32_t cols, const float* w, uint8_t* q,
                          uint8_t* scales);

/* ---- the layer, step by step ------------------------------------------- */

/* RMSNorm of m bf16 rows of width h with bf16 weight w -> bf16 rows y. */
void orc_rmsnorm(int32_t m, int32_t h, const uint16_t* x, const uint16_t* w,
                 float eps, uint16_t* y);
/* Router: logits[t,e] = sum_h y[t,h] G[e,h]; s = sigmoid(logits);
 * selection = top-k of s + bias (ties to the lower expert); weights =
 * routed_scale * s_sel / sum(s_sel).  margin[t] = b_(k) - b_(k+1) (or +inf
 * when k == E). Any output pointer may be NULL except ids. */
void orc_router(int32_t m, int32_t h, int32_t e, int32_t k, const uint16_t* y,
                const uint16_t* gate_w, const float* bias, float routed_scale,
                double* logits, int32_t* ids, double* wts, double* margin);
/* Canonical token->expert plan: counts[E]; row[t*k+j] = the row of pair (t,j)
 * when the m*k pairs are listed by expert ascending, then token ascending. */
void orc_plan(int32_t m, int32_t e, int32_t k, const int32_t* ids,
              int32_t* counts, int32_t* row);
/* The two halves of one expert for one token (orc_expert_fmt is the two in
 * turn).  up: hv [2I] = x . W13^T in double, habs [2I] (may be NULL) the
 * sums of |x_k w_nk| over the contraction, av [I] = fp32(SiLU(g) u) held in
 * double, a8 [I] / a8s [I/32] its MXFP8.  down: y [H] = a8 . W2^T. */
void orc_expert_up(int32_t h, int32_t inter, int32_t fmt, const uint8_t* x8,
                   const uint8_t* x8s, const uint8_t* w13, const uint8_t* w13_s,
                   double* hv, double* habs, double* av, uint8_t* a8, uint8_t* a8s);
void orc_expert_down(int32_t h, int32_t inter, int32_t fmt, const uint8_t* a8,
                     const uint8_t* a8s, const uint8_t* w2, const uint8_t* w2_s,
                     double* y);
/* One expert on one token: x8/x8s (H bytes, H/32 codes) -> y[H] (double);
 * a8/a8s (may be NULL) receive the quantised SiLU*up intermediate. */
void orc_expert(int32_t h, int32_t inter, const uint8_t* x8,
                const uint8_t* x8s, const uint8_t* w13, const uint8_t* w13_s,
                const uint8_t* w2, const uint8_t* w2_s, double* y, uint8_t* a8,
                uint8_t* a8s);
/* The same for weights in format fmt (ORC_FMT_E4M3 or ORC_FMT_MXFP4). */
void orc_expert_fmt(int32_t h, int32_t inter, int32_t fmt, const uint8_t* x8,
                    const uint8_t* x8s, const uint8_t* w13, const uint8_t* w13_s,
                    const uint8_t* w2, const uint8_t* w2_s, double* y,
                    uint8_t* a8, uint8_t* a8s);
/* The whole layer for m token rows.  Outputs other than out may be NULL:
 * normed [m,H] bf16, x8 [m,H], x8s [m,H/32], logits [m,E], ids [m,k],
 * wts [m,k], out_f64 [m,H] (the sum before its bf16 rounding), out [m,H] bf16.
 * Returns 0, or -1 on bad dimensions / allocation failure. */
/* One token's output from its k picked experts' outputs y_routed [k][H]
 * (weights wts [k], selection order) and the shared expert's y_shared [H]:
 * out_f64 [H] the sum in double, out [H] its bf16 (either may be NULL). */
void orc_combine(int32_t k, int32_t h, const double* wts, const double* y_routed,
                 const double* y_shared, double* out_f64, uint16_t* out);
int32_t orc_layer(const orc_dims* d, int32_t m, const uint16_t* x,
                  const uint16_t* norm_w, const uint16_t* gate_w,
                  const float* bias, const uint8_t* w13, const uint8_t* w13_s,
                  const uint8_t* w2, const uint8_t* w2_s, const uint8_t* sgu,
                  const uint8_t* sgu_s, const uint8_t* sw2,
                  const uint8_t* sw2_s, uint16_t* normed, uint8_t* x8,
                  uint8_t* x8s, double* logits, int32_t* ids, double* wts,
                  double* out_f64, uint16_t* out);

/* The hyper-connection residual fold around the FFN seam: residual and
 * residual_out bf16 [m, 4, H], part bf16 [m, H], post [m, 4], res [m, 4, 4]
 * (res[i][j]: output stream i, input stream j), pre [m, 4]; x bf16 [m, H]
 * the FFN's input row. */
void orc_hc_fold(int32_t m, int32_t h, const uint16_t* part, const uint16_t* residual,
                 const float* post, const float* res, const float* pre,
                 uint16_t* residual_out, uint16_t* x);
/* The attention seam's MXFP8 scale code of a 32-group's amax: vLLM's ROCm
 * MXFP8 code, clamp(ceil(log2(amax / 448)) + 127, 0, 254) with amax floored
 * at FLT_MIN (the same rule as orc_mx_code). */
int32_t orc_vllm_mx_code(double amax);
/* The attention seam's norm + MXFP8 (store_x8): x bf16 [m, H], w bf16 [H]
 * -> x8 [m, H] E4M3, x8s [m, H/32]. */
void orc_attn_x8(int32_t m, int32_t h, const uint16_t* x, const uint16_t* w, float eps,
                 uint8_t* x8, uint8_t* x8s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ORACLE_H */
