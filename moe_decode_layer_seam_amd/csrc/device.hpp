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
// permutations, 4 and 8 a pair of DPP row shifts with bank masks, larger
// masks go through ds_bpermute (device page, xshfl).
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

// Sum over the whole wave (every lane receives it).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += xor_lane(v, m);
  return v;
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

}  // namespace moe
