// hc.hip -- the seam around the MoE, upstream of its norm:
//   hc_fold: the attention output folded into the four-stream
//            hyper-connection residual with the attention seam's mixes, and
//            the FFN's input row combined from the new streams;
//   attn_x8: the attention seam's norm output quantised with vLLM's MXFP8
//            code (the device page's mx_code) and clamped to the E4M3 range
//            (the attention's input).
//
// Pages: "vllm.models.deepseek_v41.amd.mono.layer" run_ffn (the attention's
// partials summed and folded into the residual), store_x8 (amax over 32
// columns, vllm_mx_code, 2^(127 - code), clamp_fp8, fp8_pack4);
// "vllm.models.deepseek_v41.amd.mono.runner" DSV41MonoLayer.ffn (residual
// [M, 4, 5120] bf16, post_mix [M, 4, 1], res_mix [M, 4, 4], pre_mix [M, 4]).
//
// Both move a few MB at most: at these sizes they are bound by latency, not
// by HBM bandwidth.
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// bf16 of a double, rounded to nearest even in one step: the double is
// first rounded to fp32 toward zero with the lost bits kept as a sticky low
// bit (round to odd), which makes the following fp32 -> bf16 rounding exact.
__device__ __forceinline__ uint32_t f64_to_bf16(double v) {
  float f = __double2float_rz(v);
  if ((double)f != v) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f32_to_bf16(f);
}

// Token t = blockIdx.y, columns [2 c, 2 c + 2) with c = blockIdx.x * 256 +
// threadIdx.x (two columns a thread keeps each thread's chain of double
// operations short; the kernel is latency-bound at these sizes).  New stream
// i = bf16(sum_j res[i][j] r_j + post[i] part), the input row
// bf16(sum_i pre[i] r'_i) over the rounded streams; every sum in double in
// that order.  residual_out may be residual itself: a thread reads its
// columns of all four streams before it writes them.
__global__ __launch_bounds__(kThreads) void hc_fold_kernel(int H, const uint16_t* __restrict__ part,
                                                           const uint16_t* residual, const float* __restrict__ post,
                                                           const float* __restrict__ res,
                                                           const float* __restrict__ pre, uint16_t* residual_out,
                                                           uint16_t* __restrict__ x) {
  const int t = blockIdx.y;
  const int col = 2 * (blockIdx.x * kThreads + threadIdx.x);
  if (col >= H) return;
  const size_t row = (size_t)t * H + col;
  uint32_t rv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) rv[j] = *reinterpret_cast<const uint32_t*>(residual + ((size_t)t * 4 + j) * H + col);
  const uint32_t pv = *reinterpret_cast<const uint32_t*>(part + row);
  double mr[16], mp[4], mx[4];
#pragma unroll
  for (int k = 0; k < 16; ++k) mr[k] = (double)res[t * 16 + k];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mp[i] = (double)post[t * 4 + i];
    mx[i] = (double)pre[t * 4 + i];
  }
  uint32_t out[4] = {}, xo = 0;
#pragma unroll
  for (int z = 0; z < 2; ++z) {
    double r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = (double)bf16_to_f32(z ? (rv[j] >> 16) : (rv[j] & 0xFFFFu));
    const double p = (double)bf16_to_f32(z ? (pv >> 16) : (pv & 0xFFFFu));
    double xs = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = acc + mr[i * 4 + j] * r[j];
      acc = acc + mp[i] * p;
      const uint32_t b = f64_to_bf16(acc);
      out[i] |= b << (16 * z);
      xs = xs + mx[i] * (double)bf16_to_f32(b);
    }
    xo |= f64_to_bf16(xs) << (16 * z);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(residual_out + ((size_t)t * 4 + i) * H + col) = out[i];
  *reinterpret_cast<uint32_t*>(x + row) = xo;
}

// Token t = blockIdx.x: the RMSNorm chain of the seam (double sum of
// squares, r rounded once to fp32, two fp32 products) without the bf16 step,
// then per 32 columns (4 lanes of 8) vLLM's MXFP8 code of the amax (the
// device page's mx_code: the smallest code whose range 448 * 2^(code - 127)
// holds the amax, e8m0_code), the values scaled by 2^(127 - code), clamped to
// +-448 as clamp_fp8 does, and rounded to E4M3.
template <int CPT>
__global__ __launch_bounds__(kThreads) void attn_x8_kernel(int H, const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ w, float eps,
                                                           uint8_t* __restrict__ x8, uint8_t* __restrict__ x8s) {
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = blockIdx.x;
  u32x4 xv[CPT], wv[CPT];
  bool live[CPT];
  int col[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    col[q] = 8 * tid + 2048 * q;
    live[q] = col[q] < H;
    xv[q] = live[q] ? *reinterpret_cast<const u32x4*>(x + (size_t)t * H + col[q]) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int q = 0; q < CPT; ++q)
    wv[q] = live[q] ? *reinterpret_cast<const u32x4*>(w + col[q]) : u32x4{0u, 0u, 0u, 0u};
  double ss = 0.0;
#pragma unroll
  for (int q = 0; q < CPT; ++q) ss = add_squares8(ss, xv[q]);
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const double tot = red[0] + red[1] + red[2] + red[3];
  const float r = (float)(1.0 / sqrt(tot / (double)H + (double)eps));
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    float y[8];
#pragma unroll
    for (int z = 0; z < 8; ++z) {
      const uint32_t xb = (z & 1) ? (xv[q][z >> 1] >> 16) : (xv[q][z >> 1] & 0xFFFFu);
      const uint32_t wb = (z & 1) ? (wv[q][z >> 1] >> 16) : (wv[q][z >> 1] & 0xFFFFu);
      const float xr = bf16_to_f32(xb) * r;
      y[z] = xr * bf16_to_f32(wb);
    }
    float amax = 0.0f;
#pragma unroll
    for (int z = 0; z < 8; ++z) amax = fmaxf(amax, fabsf(y[z]));
    amax = group_max(amax, 4);
    const int code = e8m0_code(amax);
    const float mul = mx_mul(code);
    float v[8];
#pragma unroll
    for (int z = 0; z < 8; ++z) v[z] = fminf(fmaxf(y[z] * mul, -448.0f), 448.0f);
    if (live[q]) {
      u32x2 qv;
      qv[0] = fp8x4(v[0], v[1], v[2], v[3]);
      qv[1] = fp8x4(v[4], v[5], v[6], v[7]);
      *reinterpret_cast<u32x2*>(x8 + (size_t)t * H + col[q]) = qv;
      if ((lane & 3) == 0) x8s[(size_t)t * (H / 32) + col[q] / 32] = (uint8_t)code;
    }
  }
}

}  // namespace

hipError_t launch_hc_fold(int m, int H, const uint16_t* part, const uint16_t* residual, const float* post,
                          const float* res, const float* pre, uint16_t* residual_out, uint16_t* x, hipStream_t st) {
  const dim3 grid((H / 2 + kThreads - 1) / kThreads, m);
  hipLaunchKernelGGL(hc_fold_kernel, grid, dim3(kThreads), 0, st, H, part, residual, post, res, pre, residual_out, x);
  return hipGetLastError();
}

hipError_t launch_attn_x8(int m, int H, const uint16_t* x, const uint16_t* w, float eps, uint8_t* x8, uint8_t* x8s,
                          hipStream_t st) {
  const dim3 grid(m), block(kThreads);
  switch ((H + 2047) / 2048) {
    case 1: hipLaunchKernelGGL(attn_x8_kernel<1>, grid, block, 0, st, H, x, w, eps, x8, x8s); break;
    case 2: hipLaunchKernelGGL(attn_x8_kernel<2>, grid, block, 0, st, H, x, w, eps, x8, x8s); break;
    case 3: hipLaunchKernelGGL(attn_x8_kernel<3>, grid, block, 0, st, H, x, w, eps, x8, x8s); break;
    case 4: hipLaunchKernelGGL(attn_x8_kernel<4>, grid, block, 0, st, H, x, w, eps, x8, x8s); break;
    case 5: hipLaunchKernelGGL(attn_x8_kernel<5>, grid, block, 0, st, H, x, w, eps, x8, x8s); break;
    case 6: hipLaunchKernelGGL(attn_x8_kernel<6>, grid, block, 0, st, H, x, w, eps, x8, x8s); break;
    case 7: hipLaunchKernelGGL(attn_x8_kernel<7>, grid, block, 0, st, H, x, w, eps, x8, x8s); break;
    default: hipLaunchKernelGGL(attn_x8_kernel<8>, grid, block, 0, st, H, x, w, eps, x8, x8s); break;
  }
  return hipGetLastError();
}

}  // namespace moe
