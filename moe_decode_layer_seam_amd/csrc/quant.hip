// quant.hip -- weight preparation: fp32 [rows, cols] -> E4M3 with one E8M0
// code per 32 x 32 block ([rows/32, cols/32] row-major), the layout of the
// expert tensors (page "vllm.models.deepseek_v41.amd.mono.runner",
// MonoLayerWeights.check: 32 x 32 E8M0 blocks).  Code per block as mx_code,
// values rounded to nearest even after the 2^(127 - code) scaling as
// fp8_pack4 (page "vllm.models.deepseek_v41.amd.mono.attention.device").
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// One 32 x 32 block per 256 threads: thread -> row tid / 8, columns
// 4 (tid % 8) .. +4.
__global__ __launch_bounds__(256) void quant_weight_kernel(const float* __restrict__ w, int64_t nblocks,
                                                           int rows, int cols, uint8_t* __restrict__ q,
                                                           uint8_t* __restrict__ sc) {
  __shared__ float wmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = tid >> 3, cq = (tid & 7) * 4;
  const int rb = rows / 32, cb = cols / 32;
  for (int64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
    const int64_t mat = blk / ((int64_t)rb * cb);
    const int rem = (int)(blk % ((int64_t)rb * cb));
    const int br = rem / cb, bc = rem % cb;
    const size_t at = (size_t)mat * rows * cols + (size_t)(br * 32 + r) * cols + bc * 32 + cq;
    const float4 v = *reinterpret_cast<const float4*>(w + at);
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = group_max(amax, 64);
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    __syncthreads();
    const int code = e8m0_code(amax);
    const float mul = mx_mul(code);
    *reinterpret_cast<uint32_t*>(q + at) = fp8x4(v.x * mul, v.y * mul, v.z * mul, v.w * mul);
    if (tid == 0) sc[(size_t)mat * rb * cb + rem] = (uint8_t)code;
  }
}

// MXFP4: one row and 32 columns per 8 lanes, 4 columns per lane; codes
// [rows, cols/32], elements E2M1 two per byte, column 2i in the low nibble
// (page "vllm.models.deepseek_v41.amd.mono.runner", MonoLayerWeights.check:
// routed w13 / w2 fp4x2 with one code per row and 32 columns; codes in a
// blocked order, see the kernel).
__global__ __launch_bounds__(256) void quant_weight_fp4_kernel(const float* __restrict__ w, int64_t ngroups,
                                                               int rows, int cols, uint8_t* __restrict__ q,
                                                               uint8_t* __restrict__ sc) {
  const int cb = cols / 32, nsg = (cols + 511) / 512;
  const int64_t stride = (int64_t)gridDim.x * 32;  // groups of 32 columns per sweep
  for (int64_t grp = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3); grp < ngroups; grp += stride) {
    const int sub = threadIdx.x & 7;
    const float4 v = *reinterpret_cast<const float4*>(w + grp * 32 + 4 * sub);
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = group_max(amax, 8);
    const int code = fp4_code(amax);
    const float mul = mx_mul(code);
    const uint32_t n0 = e2m1_rne(v.x * mul), n1 = e2m1_rne(v.y * mul);
    const uint32_t n2 = e2m1_rne(v.z * mul), n3 = e2m1_rne(v.w * mul);
    *reinterpret_cast<uint16_t*>(q + grp * 16 + 2 * sub) = (uint16_t)(n0 | (n1 << 4) | (n2 << 8) | (n3 << 12));
    if (sub == 0) {
      // blocked code order [rows/16][nsg][16][16] per matrix: the codes of a
      // 16-row tile's 512-column segment are one 256-byte block
      const int64_t er = grp / cb;  // matrix * rows + row
      const int b = (int)(grp - er * cb), r = (int)(er % rows);
      const int64_t e = er / rows;
      const int64_t at = ((e * (rows / 16) + r / 16) * nsg + b / 16) * 256 + (r % 16) * 16 + b % 16;
      sc[at] = (uint8_t)code;
    }
  }
}

}  // namespace

hipError_t launch_quant_weight_fp4(const float* w, int count, int rows, int cols, uint8_t* q, uint8_t* sc,
                                   hipStream_t st) {
  if ((cols / 32) % 16) {  // a ragged last segment: its padding codes are 0
    const size_t nbytes = (size_t)count * (rows / 16) * ((cols + 511) / 512) * 256;
    const hipError_t e = hipMemsetAsync(sc, 0, nbytes, st);
    if (e != hipSuccess) return e;
  }
  // every lane of a 256-thread block stays in its 8-lane group for the loop,
  // whose trip count is uniform across the group
  const int64_t ngroups = (int64_t)count * rows * (cols / 32);
  const int64_t blocks = (ngroups + 31) / 32;
  const int grid = (int)(blocks < 16384 ? blocks : 16384);
  hipLaunchKernelGGL(quant_weight_fp4_kernel, dim3(grid), dim3(256), 0, st, w, ngroups, rows, cols, q, sc);
  return hipGetLastError();
}

hipError_t launch_quant_weight(const float* w, int count, int rows, int cols, uint8_t* q, uint8_t* sc,
                               hipStream_t st) {
  const int64_t nblocks = (int64_t)count * (rows / 32) * (cols / 32);
  const int grid = (int)(nblocks < 16384 ? nblocks : 16384);
  hipLaunchKernelGGL(quant_weight_kernel, dim3(grid), dim3(256), 0, st, w, nblocks, rows, cols, q, sc);
  return hipGetLastError();
}

}  // namespace moe
