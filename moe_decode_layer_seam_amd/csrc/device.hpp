// device.hpp -- wave-level primitives for gfx950 (CDNA4, 64-lane waves).
//
// Written for this library from the behaviour the pages document on page
// "vllm.models.deepseek_v41.amd.mono.attention.device" (xshfl / butterfly,
// mx_code, mx_mul, fp8_pack4, mfma_scaled, bf16_pair) and from the measured
// lane layout of the gfx950 scaled MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Lane exchange: value of lane (lane ^ mask).  Masks 1 and 2 are DPP quad
// permutations, 4 and 8 a pair of DPP row shifts with bank masks, 16 and 32
// permlane swaps across rows (device page, xshfl), 15 the DPP row mirror
// (31 and 63: the mirror, then the row swaps); others ds_bpermute.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xor_lane(int v, int mask) {
  switch (mask) {
    case 1:
      return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    case 2:
      return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    case 4: {
      int y = __builtin_amdgcn_update_dpp(v, v, 0x114, 0xF, 0xA, false);  // row_shr:4, banks 1,3
      return __builtin_amdgcn_update_dpp(y, v, 0x104, 0xF, 0x5, false);   // row_shl:4, banks 0,2
    }
    case 8: {
      int y = __builtin_amdgcn_update_dpp(v, v, 0x118, 0xF, 0xC, false);  // row_shr:8, banks 2,3
      return __builtin_amdgcn_update_dpp(y, v, 0x108, 0xF, 0x3, false);   // row_shl:8, banks 0,1
    }
    case 16: {
      // v_permlane16_swap: odd 16-lane rows of the first operand trade
      // places with even rows of the second
      const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
      return (int)(((threadIdx.x >> 4) & 1) ? r[0] : r[1]);
    }
    case 32: {
      // v_permlane32_swap: upper 32 lanes of the first operand trade places
      // with the lower 32 of the second
      const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
      return (int)(((threadIdx.x >> 5) & 1) ? r[0] : r[1]);
    }
    case 15:
      return __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false);  // row_mirror
    case 31: {
      // row mirror, then the 16-lane rows swapped in pairs
      const int y = __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false);
      const auto r = __builtin_amdgcn_permlane16_swap((unsigned)y, (unsigned)y, false, false);
      return (int)(((threadIdx.x >> 4) & 1) ? r[0] : r[1]);
    }
    case 63: {
      // row mirror, then rows swapped in pairs, then the halves swapped
      const int y = __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false);
      const auto r = __builtin_amdgcn_permlane16_swap((unsigned)y, (unsigned)y, false, false);
      const unsigned z = ((threadIdx.x >> 4) & 1) ? r[0] : r[1];
      const auto q = __builtin_amdgcn_permlane32_swap(z, z, false, false);
      return (int)(((threadIdx.x >> 5) & 1) ? q[0] : q[1]);
    }
    default:
      return __shfl_xor(v, mask, kWave);
  }
}

__device__ __forceinline__ float xor_lane(float v, int mask) {
  return __int_as_float(xor_lane(__float_as_int(v), mask));
}

__device__ __forceinline__ double xor_lane(double v, int mask) {
  int64_t b = __double_as_longlong(v);
  int lo = xor_lane((int)(b & 0xFFFFFFFF), mask);
  int hi = xor_lane((int)(b >> 32), mask);
  return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}

// Sum over the whole wave (every lane receives it): pairs of lanes 32
// apart, then 16, ... then 1.  reduce_scatter below adds in the same tree.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) v += xor_lane(v, m);
  return v;
}

// Wave sums of NV values at once (NV a power of two <= 32), each added in
// the same tree as wave_sum.  The first log2(NV) steps halve the values a
// lane carries (it keeps one half, adds its partner's copy of that half and
// hands over the other); the rest are plain butterfly steps.  On return v[0]
// of lane l holds the sum of value l >> (6 - log2(NV)).
template <int NV, int M = kWave / 2, int H = NV / 2>
__device__ __forceinline__ void reduce_scatter(double (&v)[NV], int lane) {
  // one butterfly step per template level, so every index is a constant and
  // the values stay in registers
  if constexpr (M >= 1) {
    if constexpr (H >= 1) {
      const bool up = (lane & M) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const double keep = up ? v[H + i] : v[i];
        const double give = up ? v[i] : v[H + i];
        v[i] = keep + xor_lane(give, M);
      }
      reduce_scatter<NV, M / 2, H / 2>(v, lane);
    } else {
      v[0] += xor_lane(v[0], M);
      reduce_scatter<NV, M / 2, 0>(v, lane);
    }
  }
}

__device__ __forceinline__ float group_max(float v, int width) {
  for (int m = 1; m < width; m <<= 1) v = fmaxf(v, xor_lane(v, m));
  return v;
}

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// MXFP8 (device page: mx_code, mx_mul, fp8_pack4)
// ---------------------------------------------------------------------------

// E8M0 code of a 32-group whose largest magnitude is amax >= 0 (finite):
// the smallest c in [0, 254] with amax <= 448 * 2^(c - 127).  With
// amax = M * 2^(e - 150), M = 2^23 + mantissa, and 448 = 7 * 2^6, the
// condition reads M <= 7 * 2^(c + 29 - e); since M lies in [2^23, 2^24) the
// smallest such c is e - 8, or e - 7 when M > 7 * 2^21 (mantissa > 0x600000).
// Zero and subnormal amax (below 448 * 2^-127) give 0.
__device__ __forceinline__ int e8m0_code(float amax) {
  uint32_t u = __float_as_uint(amax);
  int e = (int)(u >> 23);
  if (e == 0) return 0;
  int c = e - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return c < 0 ? 0 : (c > 254 ? 254 : c);
}

// E8M0 code of a 32-value block of FP4 (E2M1) weights: the smallest c in
// [0, 254] with amax <= 6 * 2^(c - 127) (mx_code's rule with the FP4 maximum).
// With amax = M * 2^(e - 150) and 6 = 3 * 2^1 the condition reads
// M <= 3 * 2^(c + 24 - e); M in [2^23, 2^24) makes that c = e - 2, or e - 1
// when M > 3 * 2^22 (mantissa > 0x400000).
__device__ __forceinline__ int fp4_code(float amax) {
  uint32_t u = __float_as_uint(amax);
  int e = (int)(u >> 23);
  if (e == 0) return 0;
  int c = e - 2 + ((u & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  return c < 0 ? 0 : (c > 254 ? 254 : c);
}

// E2M1 nibble of x, round to nearest with ties to the even mantissa bit,
// |x| saturating at 6, the sign bit following x.  The midpoints of the
// magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 are .25, .75, 1.25, 1.75, 2.5, 3.5, 5;
// a tie goes to the neighbour whose code is even.
__device__ __forceinline__ uint32_t e2m1_rne(float x) {
  const float a = fabsf(x);
  uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
             : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

// 2^(127 - code) as fp32, exact for code in [0, 253] (device page, mx_mul).
__device__ __forceinline__ float mx_mul(int code) { return __uint_as_float((uint32_t)(254 - code) << 23); }

// Four fp32 (|v| <= 448) -> four E4M3 bytes, round to nearest even
// (v_cvt_pk_fp8_f32; its rounding and signed zeros were checked against the
// oracle's encoder).
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ uint32_t fp8x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// ---------------------------------------------------------------------------
// The FFN seam on one lane's 8 columns ([layer] store_normed / store_x8),
// shared by every kernel that runs it so that they give the same bits.
// ---------------------------------------------------------------------------

// ss plus the squares of 8 bf16 (4 words), in double and column order (each
// square of a bf16 is exact in double).
__device__ __forceinline__ double add_squares8(double ss, const u32x4& x) {
#pragma unroll
  for (int z = 0; z < 4; ++z) {
    const double lo = bf16_to_f32(x[z] & 0xFFFFu), hi = bf16_to_f32(x[z] >> 16);
    ss += lo * lo;
    ss += hi * hi;
  }
  return ss;
}

// The normed values of 8 columns: (x r) w, each product rounded to fp32,
// then rounded to bf16 (yb) and read back (y).
__device__ __forceinline__ void norm8(const u32x4& x, const u32x4& w, float r, float (&y)[8], uint32_t (&yb)[8]) {
#pragma unroll
  for (int z = 0; z < 8; ++z) {
    const uint32_t xb = (z & 1) ? (x[z >> 1] >> 16) : (x[z >> 1] & 0xFFFFu);
    const uint32_t wb = (z & 1) ? (w[z >> 1] >> 16) : (w[z >> 1] & 0xFFFFu);
    const float xr = bf16_to_f32(xb) * r;   // fp32 product, rounded
    const float yw = xr * bf16_to_f32(wb);  // fp32 product, rounded
    yb[z] = f32_to_bf16(yw);
    y[z] = bf16_to_f32(yb[z]);
  }
}

// acc plus the router logit's terms of 8 columns: y times the bf16 gate
// weights, in double (exact products) and column order.
__device__ __forceinline__ double add_logit8(double acc, const float (&y)[8], const u32x4& g) {
#pragma unroll
  for (int z = 0; z < 8; ++z) {
    const uint32_t gb = (z & 1) ? (g[z >> 1] >> 16) : (g[z >> 1] & 0xFFFFu);
    acc += (double)y[z] * (double)bf16_to_f32(gb);
  }
  return acc;
}

// MXFP8 of 8 values of a 32-group held by 4 consecutive lanes (all four
// call it): the group's E8M0 code, and the 8 E4M3 bytes in qv.
__device__ __forceinline__ int mx8(const float (&y)[8], u32x2& qv) {
  float amax = 0.0f;
#pragma unroll
  for (int z = 0; z < 8; ++z) amax = fmaxf(amax, fabsf(y[z]));
  amax = group_max(amax, 4);
  const int code = e8m0_code(amax);
  const float mul = mx_mul(code);
  qv[0] = fp8x4(y[0] * mul, y[1] * mul, y[2] * mul, y[3] * mul);
  qv[1] = fp8x4(y[4] * mul, y[5] * mul, y[6] * mul, y[7] * mul);
  return code;
}

// ---------------------------------------------------------------------------
// Scaled MFMA 16x16x128, E4M3 x E4M3 -> fp32 (device page, mfma_scaled).
//
// Operand layout, for one 128-byte K window starting at byte kw of a row:
// lane l serves row (A) / column (B) l % 16; lane group g = l / 16 holds the
// 16 bytes [kw + 16g, +16) in its first four registers and [kw + 64 + 16g,
// +16) in the last four.  The scale byte of lane group s applies to the
// 32-byte K block [kw + 32s, +32) of its row (A) or column (B).  The result
// lane l holds D[4 (l / 16) + v][l % 16], v = 0..3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ v4f mfma_e4m3(const v8i& a, const v8i& b, v4f c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

// E4M3 A x E2M1 B (format 4).  B's lane l serves column l % 16 with the 32
// consecutive K values [32 (l / 16), +32) of the window in its first four
// registers (value 2i in the low nibble of byte i); the other four are not
// read.  Scales as for E4M3: lane 16 kb + j holds the code of K block kb of
// row / column j.  (Measured on gfx950; a scale the compiler proves uniform
// across lanes does not reach every column, so scales are per-lane values.)
__device__ __forceinline__ v4f mfma_e4m3_e2m1(const v8i& a, const u32x4& b, v4f c, int scale_a, int scale_b) {
  v8i bb;
  bb[0] = (int)b[0]; bb[1] = (int)b[1]; bb[2] = (int)b[2]; bb[3] = (int)b[3];
  bb[4] = 0; bb[5] = 0; bb[6] = 0; bb[7] = 0;
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, c, 0, 4, 0, scale_a, 0, scale_b);
}

// The same with the B scale taken from byte SEL of its operand (opsel).
template <int SEL>
__device__ __forceinline__ v4f mfma_e4m3_e2m1_sel(const v8i& a, const u32x4& b, v4f c, int scale_a,
                                                  uint32_t scale_b) {
  v8i bb;
  bb[0] = (int)b[0]; bb[1] = (int)b[1]; bb[2] = (int)b[2]; bb[3] = (int)b[3];
  bb[4] = 0; bb[5] = 0; bb[6] = 0; bb[7] = 0;
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, c, 0, 4, 0, scale_a, SEL, (int)scale_b);
}

// 4 x 4 byte transpose across the lane groups of a wave: lane (g, j) holds
// word w with byte b = M[g][b]; it returns byte b = M[b][g], where M[h][.]
// is the word of lane (h, j).  Two exchange stages, lane groups g ^ 1 then
// g ^ 2, each keeping two bytes and taking two from the partner.
__device__ __forceinline__ uint32_t transpose4_groups(uint32_t w, int g) {
  const uint32_t p1 = (uint32_t)xor_lane((int)w, 16);
  // even g: [w0, p0, w2, p2]; odd g: [p1, w1, p3, w3]
  w = __builtin_amdgcn_perm(p1, w, (g & 1) ? 0x03070105u : 0x06020400u);
  const uint32_t p2 = (uint32_t)xor_lane((int)w, 32);
  // g & 2 == 0: [w0, w1, p0, p1]; else [p2, p3, w2, w3]
  return __builtin_amdgcn_perm(p2, w, (g & 2) ? 0x03020706u : 0x05040100u);
}

__device__ __forceinline__ v8i join(const u32x4& lo, const u32x4& hi) {
  v8i r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

// 16-byte loads; the weight stream is read once, so it is marked
// non-temporal to keep it from evicting the activations from L2.
__device__ __forceinline__ u32x4 ld16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 ld16_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------------------
// Buffer loads: a 128-bit descriptor (base, byte range) held in scalar
// registers and a 32-bit per-lane offset.  Reads at or past the range return
// zero, which is how lanes without a token row read their empty operand.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

// Non-temporal (streamed once) variant for weights read in whole cache lines.
__device__ __forceinline__ u32x4 bload16_nt(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2 /* nt */);
}

// Weight tiles are read as two full-line loads: lane (g, j) of load X holds
// row (j & 7) bytes [16 g, +16) when j < 8 and [64 + 16 g, +16) when j >= 8;
// load Y the same for rows 8..15.  Two DPP row shifts per register turn the
// pair into the scaled MFMA's operand halves of row j:
//   lo = j < 8 ? X : Y(lane - 8),   hi = j < 8 ? X(lane + 8) : Y.
__device__ __forceinline__ void lines_to_mfma(const u32x4& x, const u32x4& y, u32x4& lo, u32x4& hi) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)x[i], (int)y[i], 0x118, 0xF, 0xC, false);  // row_shr:8, lanes 8-15
    hi[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)y[i], (int)x[i], 0x108, 0xF, 0x3, false);  // row_shl:8, lanes 0-7
  }
}

__device__ __forceinline__ uint32_t bload8(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

// ---------------------------------------------------------------------------
// Data exchanged between the CUs of one launch.  The L2 of an XCD does not
// see another XCD's writes, so such data is stored with the device-coherent
// policy (sc1: written through) and loaded with it (served from beyond the
// XCD's L2); AUX = kCoherent selects it on the buffer loads below, AUX = 0
// the default policy.  A writer waits for its stores to complete
// (wait_memory) before it counts them on a device-scope counter, and a
// reader issues its loads only after it has seen the count.
// ---------------------------------------------------------------------------
constexpr int kCoherent = 16;  // sc1
// Activations a launch made itself and handed over inside one XCD (the
// persistent launch's a8, values and codes): with sc0, from the XCD's L2.
// They are read only after a barrier of the XCD's blocks that follows every
// store of them, by CUs that have not read those lines before in the launch,
// so no CU's own cache holds a stale copy.
constexpr int kScL2 = 1;  // sc0

template <int AUX>
__device__ __forceinline__ u32x4 bload16a(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX);
}
template <int AUX>
__device__ __forceinline__ uint32_t bload8a(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, AUX);
}
template <int AUX>
__device__ __forceinline__ uint32_t bload32a(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, AUX);
}

__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(int4* p, int4 v) {
  int* q = reinterpret_cast<int*>(p);
  store_coherent(q, v.x);
  store_coherent(q + 1, v.y);
  store_coherent(q + 2, v.z);
  store_coherent(q + 3, v.w);
}
__device__ __forceinline__ uint32_t count_arrival(uint32_t* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sets status bits of the run (bits are only ever added: the word is
// cleared by the host, moe_decode_status, never by a kernel).
__device__ __forceinline__ void flag_status(uint32_t* p, uint32_t bits) {
  (void)__hip_atomic_fetch_or(p, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every memory operation this wave issued has completed (vector
// and scalar): stores with the coherent policy are then visible to every CU.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Timeline stamp (device page, memrealtime / stamp): thread 0 of the block
// stores the 100 MHz device clock at record [block][point] (vector store).
// tl == nullptr: no timeline.
// Blocks are numbered x-fastest; records past kTlBlockCap are dropped.  The
// last point of a record holds where the block ran: the XCC id in the upper
// half, the HW_ID register (CU, shader array, SE) in the lower.
constexpr int kTlBlockCap = 1024;

__device__ __forceinline__ void stamp(uint64_t* tl, int points, int point) {
  if (tl == nullptr || threadIdx.x != 0) return;
  const uint32_t b = blockIdx.x + blockIdx.y * gridDim.x;
  if (b >= (uint32_t)kTlBlockCap) return;
  uint64_t* rec = tl + (size_t)b * points;
  rec[point] = __builtin_amdgcn_s_memrealtime();
  if (point == 0) {
    const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_REG_HW_ID, 32 bits
    const uint32_t xcc = __builtin_amdgcn_s_getreg((15 << 11) | 20);  // HW_REG_XCC_ID
    rec[points - 1] = ((uint64_t)xcc << 32) | hw;
  }
}

// Per-wave stamp: lane 0 of the calling wave stores the clock at `point`.
__device__ __forceinline__ void stamp_wave(uint64_t* tl, int points, int point) {
  if (tl == nullptr || (threadIdx.x & 63) != 0) return;
  const uint32_t b = blockIdx.x + blockIdx.y * gridDim.x;
  if (b >= (uint32_t)kTlBlockCap) return;
  tl[(size_t)b * points + point] = __builtin_amdgcn_s_memrealtime();
}

// A lane offset no buffer of this library reaches: loads through it read 0.
constexpr uint32_t kNoRow = 0x7FFFFF00u;

}  // namespace moe
