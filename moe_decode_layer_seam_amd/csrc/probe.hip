// probe.hip -- a plain streaming read of a device buffer: every byte once,
// in 128-bit non-temporal loads (the width and cache policy of the expert
// GEMMs' weight loads), sixteen loads in flight per thread.  Its rate is the
// measured HBM read peak that the weight streaming is set against, beside
// the published one.  Each block stores the XOR of the 32-bit words it read,
// so the reads cannot be dropped and the result can be checked.
//
// Shape: each block streams one contiguous range; a sweep over 4 GiB on
// MI355X (contiguous or interleaved chunks, 4-16 loads in flight, 256 or 512
// threads, 1024-4096 blocks) put this shape at the top, 7.1 TB/s.
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 16;

// Block b reads words [b per, (b + 1) per) of the n 16-byte words, per being
// n / B rounded down to whole chunks of kProbeThreads * kProbeUnroll words
// (thread t: word t of each kProbeThreads-word row); the words past B per
// are read one a thread, spread over all blocks.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ p, uint64_t n,
                                                                   uint32_t* __restrict__ sink) {
  constexpr uint64_t chunk = (uint64_t)kProbeThreads * kProbeUnroll;
  __shared__ uint32_t part[kProbeThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const uint64_t B = gridDim.x, per = n / B / chunk * chunk;
  uint32_t acc = 0;
  const uint64_t b0 = (uint64_t)blockIdx.x * per;
  for (uint64_t base = b0; base < b0 + per; base += chunk) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) v[k] = __builtin_nontemporal_load(p + base + k * kProbeThreads + tid);
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (uint64_t i = B * per + (uint64_t)blockIdx.x * kProbeThreads + tid; i < n; i += B * kProbeThreads) {
    const u32x4 v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int m = 1; m < 64; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
  if (lane == 0) part[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / 64; ++w) x ^= part[w];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(MOE_DECODE_PROBE_BLOCKS), dim3(kProbeThreads), 0, st,
                     static_cast<const u32x4*>(buf), (uint64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace moe
