/*
 * moe_oracle.c -- the CPU oracle of the small-batch decode MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h): the checker the HIP path is
 * compared with.  Plain C, single-threaded, double precision; compiled with
 * -ffp-contract=off so that no multiply-add is fused behind the reader's back.
 *
 * Page references:
 *   [layer]  "vllm.models.deepseek_v41.amd.mono.layer"
 *   [runner] "vllm.models.deepseek_v41.amd.mono.runner"
 *   [device] "vllm.models.deepseek_v41.amd.mono.attention.device"
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16                                                                     */
/* ------------------------------------------------------------------------ */

double orc_bf16_value(uint16_t b) {
  /* A bf16 is the upper half of an IEEE binary32. */
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Round a non-negative finite double to the nearest integer, ties to even. */
static double round_half_even(double r) {
  double fl = floor(r);
  double frac = r - fl; /* exact: r and fl are close */
  if (frac > 0.5) return fl + 1.0;
  if (frac < 0.5) return fl;
  return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

uint16_t orc_bf16_rne(double v) {
  /* bf16: 8 significant bits (7 stored), exponent range of binary32,
   * subnormals down to 2^-133.  The nearest value is n * quantum with n an
   * integer, where quantum is the spacing of bf16 values around |v|. */
  if (isnan(v)) return 0x7FC0;
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  uint16_t mag;
  if (a == 0.0) {
    mag = 0;
  } else {
    int e;
    (void)frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
    int qexp = (e - 1 >= -126) ? (e - 1) - 7 : -133;
    double n = round_half_even(ldexp(a, -qexp)); /* exact scaling */
    double r = ldexp(n, qexp);
    if (r >= ldexp(1.0, 128)) {
      mag = 0x7F80; /* overflow to infinity */
    } else {
      float f = (float)r; /* exact: r has at most 8 significant bits */
      uint32_t bits;
      memcpy(&bits, &f, sizeof bits);
      mag = (uint16_t)(bits >> 16);
    }
  }
  return (uint16_t)(mag | (neg ? 0x8000 : 0));
}

/* ------------------------------------------------------------------------ */
/* E4M3 (float8_e4m3fn) and E8M0                                            */
/* ------------------------------------------------------------------------ */

double orc_e4m3_value(uint8_t b) {
  /* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
   * subnormal (m * 2^-9); S.1111.111 is NaN; no infinities. */
  int s = b >> 7, e = (b >> 3) & 0xF, m = b & 7;
  double v;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Lookup tables filled once, at load time, from the closed forms above:
 * E4M3[b] = orc_e4m3_value(b) and POW2[c] = 2^(c - 127).  They only spare the
 * quantisers and the dot products a call to ldexp per element. */
static double E4M3[256];
static double POW2[256];
static double E2M1[16];

__attribute__((constructor)) static void orc_tables(void) {
  for (int b = 0; b < 256; ++b) {
    E4M3[b] = orc_e4m3_value((uint8_t)b);
    POW2[b] = ldexp(1.0, b - 127);
  }
  for (int n = 0; n < 16; ++n) E2M1[n] = orc_e2m1_value((uint8_t)n);
}

uint8_t orc_e4m3_rne(double v) {
  /* Nearest representable magnitude with ties to the even code.  The 127
   * non-negative finite codes 0x00..0x7E increase with their value, so the
   * neighbours of |v| are found by a search over the code order. */
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  if (a > 448.0) a = 448.0; /* clamp to the largest finite E4M3 */
  /* lo = the largest code in [0, 0x7E] whose value is <= a, by bisection:
   * try to advance lo by 64, 32, ..., 1 while staying at or below a. */
  int lo = 0;
  for (int step = 64; step >= 1; step /= 2)
    if (lo + step <= 0x7E && E4M3[lo + step] <= a) lo += step;
  int code = lo;
  if (lo < 0x7E) {
    double dlo = a - E4M3[lo];
    double dhi = E4M3[lo + 1] - a;
    if (dhi < dlo || (dhi == dlo && (lo & 1))) code = lo + 1;
  }
  return (uint8_t)(code | (neg ? 0x80 : 0));
}

int32_t orc_mx_code(double amax) {
  /* [device] mx_code: clamp(ceil(log2(amax / 448)) + 127, 0, 254).  Read as
   * the smallest integer c in [0, 254] with amax <= 448 * 2^(c - 127); every
   * product below is an exact power-of-two scaling in double precision. */
  for (int32_t c = 0; c < 254; ++c)
    if (amax <= ldexp(448.0, c - 127)) return c;
  return 254;
}

/* ------------------------------------------------------------------------ */
/* E2M1 (float4_e2m1fn, two per byte) and its E8M0 scale code                */
/* ------------------------------------------------------------------------ */

double orc_e2m1_value(uint8_t nibble) {
  /* [runner] MonoLayerWeights.check: the routed experts' torch.float4_e2m1fn_x2
   * (the OCP MX FP4 element): 1 sign bit, 2 exponent bits (bias 1), 1
   * mantissa bit; exponent 0 is subnormal (m * 2^-1); no infinities or NaN. */
  int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
  double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

uint8_t orc_e2m1_rne(double v) {
  /* Nearest of the eight magnitudes (codes 0..7 increase with their value),
   * ties to the code with an even (zero) mantissa bit; |v| above 6, the
   * largest, saturates; the sign bit follows v (a negative value that rounds
   * to zero gives 0x8, as for E4M3). */
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  if (a > 6.0) a = 6.0;
  int best = 0;
  double bd = a;  /* distance to code 0 (value 0) */
  for (int c = 1; c < 8; ++c) {
    double dist = fabs(a - E2M1[c]);
    if (dist < bd || (dist == bd && (c & 1) == 0)) {
      best = c;
      bd = dist;
    }
  }
  return (uint8_t)(best | (neg ? 0x8 : 0));
}

int32_t orc_fp4_code(double amax) {
  /* The E8M0 code of a 32-value block of FP4 weights: the same rule as
   * [device] mx_code with the FP4 maximum 6 in place of 448, i.e. the
   * smallest integer c in [0, 254] with amax <= 6 * 2^(c - 127), so that no
   * element of the block needs clamping. */
  for (int32_t c = 0; c < 254; ++c)
    if (amax <= ldexp(6.0, c - 127)) return c;
  return 254;
}

void orc_e2m1_rne_array(int64_t n, const double* v, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_rne(v[i]);
}

void orc_e4m3_rne_array(int64_t n, const double* v, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_rne(v[i]);
}

void orc_mx_code_array(int64_t n, const double* amax, int32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_mx_code(amax[i]);
}

void orc_bf16_rne_array(int64_t n, const double* v, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_rne(v[i]);
}

/* ------------------------------------------------------------------------ */
/* Quantisers                                                               */
/* ------------------------------------------------------------------------ */

void orc_mx_quant_row(int32_t n, const double* v, uint8_t* q, uint8_t* codes) {
  /* [layer] store_x8: per 32 contiguous values, amax -> code, multiplier
   * 2^(127 - code), clamp to +-448, E4M3 round-to-nearest-even. */
  for (int32_t g = 0; g < n / 32; ++g) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
      double a = fabs(v[g * 32 + i]);
      if (a > amax) amax = a;
    }
    int32_t c = orc_mx_code(amax);
    codes[g] = (uint8_t)c;
    for (int i = 0; i < 32; ++i)
      q[g * 32 + i] = orc_e4m3_rne(v[g * 32 + i] * POW2[254 - c]); /* 2^(127-c) */
  }
}

void orc_quant_weight(int32_t rows, int32_t cols, const float* w, uint8_t* q,
                      uint8_t* scales) {
  /* One E8M0 code per 32 x 32 block, scales laid out [rows/32, cols/32]
   * row-major ([runner] MonoLayerWeights.check: sgu_s [2 Is/32, H/32],
   * sw2_s [H/32, Is/32]; AttnWeights.check: wqkv_scale [56, 160]).
   * Pass 1 finds every block's amax, pass 2 encodes; both walk the matrix
   * row by row. */
  int32_t cb = cols / 32;
  double* amax = (double*)calloc((size_t)(rows / 32) * cb, sizeof(double));
  for (int32_t r = 0; r < rows; ++r)
    for (int32_t c = 0; c < cols; ++c) {
      double a = fabs((double)w[(size_t)r * cols + c]);
      double* m = &amax[(size_t)(r / 32) * cb + c / 32];
      if (a > *m) *m = a;
    }
  for (size_t b = 0; b < (size_t)(rows / 32) * cb; ++b)
    scales[b] = (uint8_t)orc_mx_code(amax[b]);
  for (int32_t r = 0; r < rows; ++r)
    for (int32_t c = 0; c < cols; ++c) {
      int32_t code = scales[(size_t)(r / 32) * cb + c / 32];
      size_t at = (size_t)r * cols + c;
      q[at] = orc_e4m3_rne((double)w[at] * POW2[254 - code]); /* 2^(127-code) */
    }
  free(amax);
}

size_t orc_fp4_code_index(int32_t cols, int32_t r, int32_t b) {
  /* Blocked order of the MXFP4 codes: [rows/16][ceil(cols/512)][16][16]; the
   * 16 x 16 codes of a 16-row, 512-column tile are one contiguous 256-byte
   * block, row-major inside (the pages keep these codes in a shuffled order
   * of their own too: [runner] MonoLayerWeights, w13_s "shuffle_scale"). */
  int32_t nsg = (cols + 511) / 512;
  return ((size_t)(r / 16) * nsg + (size_t)(b / 16)) * 256 + (size_t)(r % 16) * 16 + (size_t)(b % 16);
}

void orc_quant_weight_fp4(int32_t rows, int32_t cols, const float* w, uint8_t* q,
                          uint8_t* scales) {
  /* MXFP4 of a [rows, cols] fp32 weight: one E8M0 code per row and 32
   * consecutive columns, elements E2M1(w * 2^(127 - code)), two per byte:
   * column 2i in the low nibble, column 2i + 1 in the high one ([runner]
   * MonoLayerWeights.check: w13 [E, 2I, H/2] fp4x2, w2 [E, H, I/2]).  Codes
   * in the blocked order of orc_fp4_code_index; padding codes are 0. */
  int32_t cb = cols / 32;
  memset(scales, 0, (size_t)(rows / 16) * ((cols + 511) / 512) * 256);
  for (int32_t r = 0; r < rows; ++r)
    for (int32_t b = 0; b < cb; ++b) {
      const float* src = w + (size_t)r * cols + (size_t)b * 32;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i)
        if (fabs((double)src[i]) > amax) amax = fabs((double)src[i]);
      int32_t code = orc_fp4_code(amax);
      scales[orc_fp4_code_index(cols, r, b)] = (uint8_t)code;
      uint8_t* dst = q + (size_t)r * (cols / 2) + (size_t)b * 16;
      for (int i = 0; i < 16; ++i) {
        uint8_t lo = orc_e2m1_rne((double)src[2 * i] * POW2[254 - code]);
        uint8_t hi = orc_e2m1_rne((double)src[2 * i + 1] * POW2[254 - code]);
        dst[i] = (uint8_t)(lo | (hi << 4));
      }
    }
}

/* Dequantised E4M3 element with its E8M0 code: value * 2^(code - 127). */
static double mx_value(uint8_t q, uint8_t code) {
  return E4M3[q] * POW2[code]; /* exact: a power-of-two scaling */
}

/* Weight element (n, k) of an [N, K] expert matrix, dequantised, in either
 * routed format: E4M3 with 32 x 32 blocks (codes [N/32, K/32]) or MXFP4 with
 * 1 x 32 blocks (two elements per byte, codes in blocked order). */
static double weight_value(int32_t fmt, const uint8_t* w, const uint8_t* ws,
                           int32_t K, int32_t n, int32_t k) {
  if (fmt == ORC_FMT_MXFP4) {
    uint8_t byte = w[(size_t)n * (K / 2) + k / 2];
    uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 0xF);
    return E2M1[nib] * POW2[ws[orc_fp4_code_index(K, n, k / 32)]];
  }
  return mx_value(w[(size_t)n * K + k], ws[(size_t)(n / 32) * (K / 32) + k / 32]);
}

/* ------------------------------------------------------------------------ */
/* RMSNorm                                                                  */
/* ------------------------------------------------------------------------ */

static float round_f32(double v) { return (float)v; }

void orc_rmsnorm(int32_t m, int32_t h, const uint16_t* x, const uint16_t* w,
                 float eps, uint16_t* y) {
  /* The norm feeding the MoE ([layer] run_ffn: the FFN seam's norm, its row
   * stored as bf16 by store_normed).  The pages name the norm but do not
   * print its arithmetic; the reading taken: the sum of squares in double,
   * r = 1/sqrt(ss/H + eps) rounded once to fp32, then two fp32 products
   * (x * r, then * w), then one rounding to bf16. */
  for (int32_t t = 0; t < m; ++t) {
    const uint16_t* xr = x + (size_t)t * h;
    double ss = 0.0;
    for (int32_t i = 0; i < h; ++i) {
      double v = orc_bf16_value(xr[i]);
      ss += v * v;
    }
    float r = round_f32(1.0 / sqrt(ss / (double)h + (double)eps));
    for (int32_t i = 0; i < h; ++i) {
      float xr_ = round_f32(orc_bf16_value(xr[i]) * (double)r);
      float yw = round_f32((double)xr_ * orc_bf16_value(w[i]));
      y[(size_t)t * h + i] = orc_bf16_rne((double)yw);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Router                                                                   */
/* ------------------------------------------------------------------------ */

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

void orc_router(int32_t m, int32_t h, int32_t e, int32_t k, const uint16_t* y,
                const uint16_t* gate_w, const float* bias, float routed_scale,
                double* logits, int32_t* ids, double* wts, double* margin) {
  /* gate_w [E, H] bf16 and bias [E] f32, the e_score_correction_bias
   * ([runner] MonoLayerWeights).  Scores are sigmoids of the logits; the bias
   * only ranks the experts; the picked experts' scores are renormalised to
   * sum to one and multiplied by routed_scale. */
  double* l = (double*)malloc(sizeof(double) * (size_t)e);
  double* s = (double*)malloc(sizeof(double) * (size_t)e);
  double* b = (double*)malloc(sizeof(double) * (size_t)e);
  char* taken = (char*)malloc((size_t)e);
  for (int32_t t = 0; t < m; ++t) {
    for (int32_t x = 0; x < e; ++x) {
      double acc = 0.0;
      for (int32_t i = 0; i < h; ++i)
        acc += orc_bf16_value(y[(size_t)t * h + i]) *
               orc_bf16_value(gate_w[(size_t)x * h + i]);
      l[x] = acc;
      s[x] = sigmoid(acc);
      b[x] = s[x] + (double)bias[x];
      taken[x] = 0;
      if (logits) logits[(size_t)t * e + x] = acc;
    }
    /* k rounds of "take the largest b not yet taken; on equal b the lower
     * expert index first". */
    double ssum = 0.0, last = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t x = 0; x < e; ++x)
        if (!taken[x] && (best < 0 || b[x] > b[best])) best = x;
      taken[best] = 1;
      ids[(size_t)t * k + j] = best;
      ssum += s[best];
      last = b[best];
    }
    if (margin) {
      int32_t next = -1;
      for (int32_t x = 0; x < e; ++x)
        if (!taken[x] && (next < 0 || b[x] > b[next])) next = x;
      margin[t] = (next < 0) ? INFINITY : last - b[next];
    }
    if (wts)
      for (int32_t j = 0; j < k; ++j)
        wts[(size_t)t * k + j] =
            (double)routed_scale * s[ids[(size_t)t * k + j]] / ssum;
  }
  free(l);
  free(s);
  free(b);
  free(taken);
}

void orc_plan(int32_t m, int32_t e, int32_t k, const int32_t* ids,
              int32_t* counts, int32_t* row) {
  /* Every (token, pick) pair once, grouped by expert in ascending expert
   * order and within an expert by ascending token. */
  int32_t r = 0;
  for (int32_t x = 0; x < e; ++x) {
    counts[x] = 0;
    for (int32_t t = 0; t < m; ++t)
      for (int32_t j = 0; j < k; ++j)
        if (ids[(size_t)t * k + j] == x) {
          row[(size_t)t * k + j] = r++;
          counts[x] += 1;
        }
  }
}

/* ------------------------------------------------------------------------ */
/* Experts and the combine                                                  */
/* ------------------------------------------------------------------------ */

void orc_expert_up(int32_t h, int32_t inter, int32_t fmt, const uint8_t* x8,
                   const uint8_t* x8s, const uint8_t* w13, const uint8_t* w13_s,
                   double* hv, double* habs, double* av, uint8_t* a8, uint8_t* a8s) {
  /* w13 [2I, H]: rows [0, I) the gate, rows [I, 2I) the up projection, in
   * the weight format fmt (see weight_value).  h = x . W13^T with both
   * operands dequantised; habs (if given) = sum over the contraction of
   * |x_k w_nk|, the magnitude the sum is taken over. */
  double* xd = (double*)malloc(sizeof(double) * (size_t)h);
  for (int32_t i = 0; i < h; ++i) xd[i] = mx_value(x8[i], x8s[i / 32]);
  for (int32_t n = 0; n < 2 * inter; ++n) {
    double acc = 0.0, mag = 0.0;
    for (int32_t i = 0; i < h; ++i) {
      double p = xd[i] * weight_value(fmt, w13, w13_s, h, n, i);
      acc += p;
      mag += fabs(p);
    }
    hv[n] = acc;
    if (habs) habs[n] = mag;
  }
  /* a = SiLU(gate) * up, held as fp32, then MXFP8 along the intermediate. */
  for (int32_t i = 0; i < inter; ++i) {
    double g = hv[i], u = hv[inter + i];
    av[i] = (double)round_f32(g * sigmoid(g) * u);
  }
  orc_mx_quant_row(inter, av, a8, a8s);
  free(xd);
}

void orc_expert_down(int32_t h, int32_t inter, int32_t fmt, const uint8_t* a8,
                     const uint8_t* a8s, const uint8_t* w2, const uint8_t* w2_s,
                     double* y) {
  /* y = a . W2^T with a the dequantised MXFP8 intermediate; w2 [H, I]. */
  for (int32_t n = 0; n < h; ++n) {
    double acc = 0.0;
    for (int32_t i = 0; i < inter; ++i)
      acc += mx_value(a8[i], a8s[i / 32]) * weight_value(fmt, w2, w2_s, inter, n, i);
    y[n] = acc;
  }
}

void orc_expert_fmt(int32_t h, int32_t inter, int32_t fmt, const uint8_t* x8,
                    const uint8_t* x8s, const uint8_t* w13, const uint8_t* w13_s,
                    const uint8_t* w2, const uint8_t* w2_s, double* y,
                    uint8_t* a8, uint8_t* a8s) {
  /* One token through one expert: the up projection with SiLU * up and
   * its MXFP8, then the down projection. */
  double* hv = (double*)malloc(sizeof(double) * 2 * (size_t)inter);
  double* av = (double*)malloc(sizeof(double) * (size_t)inter);
  uint8_t* q = (uint8_t*)malloc((size_t)inter);
  uint8_t* qc = (uint8_t*)malloc((size_t)inter / 32);
  orc_expert_up(h, inter, fmt, x8, x8s, w13, w13_s, hv, NULL, av, q, qc);
  orc_expert_down(h, inter, fmt, q, qc, w2, w2_s, y);
  if (a8) memcpy(a8, q, (size_t)inter);
  if (a8s) memcpy(a8s, qc, (size_t)inter / 32);
  free(hv);
  free(av);
  free(q);
  free(qc);
}

void orc_expert(int32_t h, int32_t inter, const uint8_t* x8,
                const uint8_t* x8s, const uint8_t* w13, const uint8_t* w13_s,
                const uint8_t* w2, const uint8_t* w2_s, double* y, uint8_t* a8,
                uint8_t* a8s) {
  orc_expert_fmt(h, inter, ORC_FMT_E4M3, x8, x8s, w13, w13_s, w2, w2_s, y, a8, a8s);
}

void orc_combine(int32_t k, int32_t h, const double* wts, const double* y_routed,
                 const double* y_shared, double* out_f64, uint16_t* out) {
  /* One token's output: the picked experts' outputs weighted in selection
   * order, then the shared expert's, summed in double; one rounding to bf16
   * ([layer] run_ffn: the MoE's output row). */
  for (int32_t n = 0; n < h; ++n) {
    double acc = 0.0;
    for (int32_t j = 0; j < k; ++j) acc += wts[j] * y_routed[(size_t)j * h + n];
    acc += y_shared[n];
    if (out_f64) out_f64[n] = acc;
    if (out) out[n] = orc_bf16_rne(acc);
  }
}

int32_t orc_layer(const orc_dims* d, int32_t m, const uint16_t* x,
                  const uint16_t* norm_w, const uint16_t* gate_w,
                  const float* bias, const uint8_t* w13, const uint8_t* w13_s,
                  const uint8_t* w2, const uint8_t* w2_s, const uint8_t* sgu,
                  const uint8_t* sgu_s, const uint8_t* sw2,
                  const uint8_t* sw2_s, uint16_t* normed, uint8_t* x8,
                  uint8_t* x8s, double* logits, int32_t* ids, double* wts,
                  double* out_f64, uint16_t* out) {
  int32_t H = d->hidden, E = d->experts, K = d->topk, I = d->inter,
          Is = d->shared_inter;
  if (m < 1 || H < 32 || H % 32 || I < 32 || I % 32 || Is < 32 || Is % 32 ||
      E < 1 || K < 1 || K > E ||
      (d->routed_format != ORC_FMT_E4M3 && d->routed_format != ORC_FMT_MXFP4))
    return -1;
  size_t mh = (size_t)m * H;
  uint16_t* y = (uint16_t*)malloc(sizeof(uint16_t) * mh);
  uint8_t* q = (uint8_t*)malloc(mh);
  uint8_t* qc = (uint8_t*)malloc(mh / 32);
  double* yv = (double*)malloc(sizeof(double) * (size_t)H);
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)m * K);
  double* w = (double*)malloc(sizeof(double) * (size_t)m * K);
  double* ye = (double*)malloc(sizeof(double) * (size_t)K * H);
  double* ysh = (double*)malloc(sizeof(double) * (size_t)H);
  if (!y || !q || !qc || !yv || !sel || !w || !ye || !ysh) return -1;

  /* 1. norm -> bf16 rows; 2. MXFP8 of each bf16 row. */
  orc_rmsnorm(m, H, x, norm_w, d->rms_eps, y);
  for (int32_t t = 0; t < m; ++t) {
    for (int32_t i = 0; i < H; ++i) yv[i] = orc_bf16_value(y[(size_t)t * H + i]);
    orc_mx_quant_row(H, yv, q + (size_t)t * H, qc + (size_t)t * (H / 32));
  }
  /* 3. router on the bf16 rows. */
  orc_router(m, H, E, K, y, gate_w, bias, d->routed_scale, logits, sel, w,
             NULL);
  /* 4-5. picked experts and the shared expert; weighted sum, one rounding. */
  /* per-expert strides of the routed tensors in their format */
  int32_t fmt = d->routed_format;
  size_t w13_e = fmt == ORC_FMT_MXFP4 ? (size_t)2 * I * (H / 2) : (size_t)2 * I * H;
  size_t w13s_e = fmt == ORC_FMT_MXFP4 ? (size_t)(2 * I / 16) * ((H + 511) / 512) * 256
                                       : (size_t)(2 * I / 32) * (H / 32);
  size_t w2_e = fmt == ORC_FMT_MXFP4 ? (size_t)H * (I / 2) : (size_t)H * I;
  size_t w2s_e = fmt == ORC_FMT_MXFP4 ? (size_t)(H / 16) * ((I + 511) / 512) * 256
                                      : (size_t)(H / 32) * (I / 32);
  for (int32_t t = 0; t < m; ++t) {
    const uint8_t* xq = q + (size_t)t * H;
    const uint8_t* xc = qc + (size_t)t * (H / 32);
    for (int32_t j = 0; j < K; ++j) {
      size_t ex = (size_t)sel[(size_t)t * K + j];
      orc_expert_fmt(H, I, fmt, xq, xc, w13 + ex * w13_e, w13_s + ex * w13s_e,
                     w2 + ex * w2_e, w2_s + ex * w2s_e, ye + (size_t)j * H, NULL, NULL);
    }
    orc_expert(H, Is, xq, xc, sgu, sgu_s, sw2, sw2_s, ysh, NULL, NULL);
    orc_combine(K, H, w + (size_t)t * K, ye, ysh, out_f64 ? out_f64 + (size_t)t * H : NULL,
                out ? out + (size_t)t * H : NULL);
  }
  if (normed) memcpy(normed, y, sizeof(uint16_t) * mh);
  if (x8) memcpy(x8, q, mh);
  if (x8s) memcpy(x8s, qc, mh / 32);
  if (ids) memcpy(ids, sel, sizeof(int32_t) * (size_t)m * K);
  if (wts) memcpy(wts, w, sizeof(double) * (size_t)m * K);
  free(y);
  free(q);
  free(qc);
  free(yv);
  free(sel);
  free(w);
  free(ye);
  free(ysh);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* The seam around the MoE: the hyper-connection residual fold and the      */
/* attention seam's MXFP8 ([layer] run_ffn, store_x8; [runner] ffn)          */
/* ------------------------------------------------------------------------ */

void orc_hc_fold(int32_t m, int32_t h, const uint16_t* part, const uint16_t* residual,
                 const float* post, const float* res, const float* pre,
                 uint16_t* residual_out, uint16_t* x) {
  /* [layer] run_ffn: the attention's output (part, TP-summed) is folded into
   * the four-stream residual [m, 4, H] with the attention seam's mixes
   * ([runner] ffn: post_mix [m, 4, 1], res_mix [m, 4, 4]); the FFN's input
   * row combines the streams with pre_mix [m, 4].  The pages give the shapes,
   * not the arithmetic; the reading taken: stream i of the new residual is
   * bf16(sum_j res[i][j] r_j + post[i] part), the input row
   * bf16(sum_i pre[i] r'_i) over the stored (bf16) new streams, each sum in
   * double in the order written, one rounding. */
  for (int32_t t = 0; t < m; ++t) {
    const uint16_t* r = residual + (size_t)t * 4 * h;
    uint16_t* ro = residual_out + (size_t)t * 4 * h;
    const float* po = post + (size_t)t * 4;
    const float* rm = res + (size_t)t * 16;
    const float* pr = pre + (size_t)t * 4;
    for (int32_t c = 0; c < h; ++c) {
      double rv[4];
      for (int j = 0; j < 4; ++j) rv[j] = orc_bf16_value(r[(size_t)j * h + c]);
      const double pv = orc_bf16_value(part[(size_t)t * h + c]);
      double xs = 0.0;
      for (int i = 0; i < 4; ++i) {
        double acc = 0.0;
        for (int j = 0; j < 4; ++j) acc += (double)rm[i * 4 + j] * rv[j];
        acc += (double)po[i] * pv;
        const uint16_t b = orc_bf16_rne(acc);
        ro[(size_t)i * h + c] = b;
        xs += (double)pr[i] * orc_bf16_value(b);
      }
      x[(size_t)t * h + c] = orc_bf16_rne(xs);
    }
  }
}

int32_t orc_vllm_mx_code(double amax) {
  /* [layer] store_x8 quantises with vLLM's MXFP8 code of the group's amax;
   * [device] mx_code is that code, named there as vLLM's ROCm MXFP8 scale
   * code: clamp(ceil(log2(amax / 448)) + 127, 0, 254), amax floored at
   * FLT_MIN.  Read as the smallest integer c in [0, 254] with
   * amax <= 448 * 2^(c - 127) (exact power-of-two scalings in double); the
   * floor at FLT_MIN only keeps the logarithm finite and yields 0 for every
   * amax below 448 * 2^-127, the all-zero group included. */
  for (int32_t c = 0; c < 254; ++c)
    if (amax <= ldexp(448.0, c - 127)) return c;
  return 254;
}

void orc_attn_x8(int32_t m, int32_t h, const uint16_t* x, const uint16_t* w, float eps,
                 uint8_t* x8, uint8_t* x8s) {
  /* [layer] store_x8: the attention seam's norm output (the RMSNorm chain of
   * orc_rmsnorm up to its fp32 product, not rounded to bf16) -> per 32
   * columns vllm_mx_code of the amax, the values scaled by 2^(127 - code),
   * clamped to +-448 (clamp_fp8; the code's bracket keeps every finite scaled
   * value inside it) and rounded to E4M3. */
  float* y = (float*)malloc(sizeof(float) * (size_t)h);
  if (!y) return;
  for (int32_t t = 0; t < m; ++t) {
    const uint16_t* xr = x + (size_t)t * h;
    double ss = 0.0;
    for (int32_t i = 0; i < h; ++i) {
      double v = orc_bf16_value(xr[i]);
      ss += v * v;
    }
    float r = round_f32(1.0 / sqrt(ss / (double)h + (double)eps));
    for (int32_t i = 0; i < h; ++i) {
      float xr_ = round_f32(orc_bf16_value(xr[i]) * (double)r);
      y[i] = round_f32((double)xr_ * orc_bf16_value(w[i]));
    }
    for (int32_t g = 0; g < h / 32; ++g) {
      double amax = 0.0;
      for (int i = 0; i < 32; ++i)
        if (fabs((double)y[g * 32 + i]) > amax) amax = fabs((double)y[g * 32 + i]);
      int32_t c = orc_vllm_mx_code(amax);
      x8s[(size_t)t * (h / 32) + g] = (uint8_t)c;
      for (int i = 0; i < 32; ++i) {
        double v = ldexp((double)y[g * 32 + i], 127 - c);
        if (v > 448.0) v = 448.0;
        if (v < -448.0) v = -448.0;
        x8[(size_t)t * h + g * 32 + i] = orc_e4m3_rne(v);
      }
    }
  }
  free(y);
}

