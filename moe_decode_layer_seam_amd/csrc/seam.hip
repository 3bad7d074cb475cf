// seam.hip -- the FFN seam and the router, one launch:
//   RMSNorm -> bf16 normed rows -> MXFP8 (x8, x8s)
//   router logits (double) -> sigmoid + bias -> top-k (sort network over
//   expert groups of 64) -> routing weights -> token->expert plan.
//
// Pages: "vllm.models.deepseek_v41.amd.mono.layer" run_ffn (the seam's norm,
// then the MoE), store_normed (the normed row, bf16), store_x8 (MXFP8 of 8
// columns per lane, amax over the 4 lanes of a 32-group, code, multiply,
// E4M3 pack); "vllm.models.deepseek_v41.amd.mono.runner" MonoLayerWeights
// (gate_w bf16 [E, H], bias f32 [E], the e_score_correction_bias);
// build_mono_ffn (expert groups of 64 for the routing sort networks).
//
// Every block computes the norm of every token (a token row is 2H bytes, so
// recomputing it is cheaper than a second launch at M <= 48) and the logits
// of its own slice of experts.  The last block to finish -- found with an
// arrival counter, no waiting -- picks the experts and writes the plan.
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// Strict total order of the router: larger biased score first, the lower
// expert index on equal scores.
__device__ __forceinline__ bool ranks_before(double b1, int e1, double b2, int e2) {
  return b1 > b2 || (b1 == b2 && e1 < e2);
}

// Bitonic sorting network over the 64 lanes, descending in the router order,
// run on NG independent groups at once.
template <int NG>
__device__ __forceinline__ void sort64(double (&b)[NG], int (&e)[NG], int lane) {
#pragma unroll
  for (int k2 = 2; k2 <= 64; k2 <<= 1) {
#pragma unroll
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      const bool up = (lane & k2) == 0;
      const bool lower = (lane & j) == 0;
      const bool keep_first = (lower == up);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        double pb = xor_lane(b[g], j);
        int pe = xor_lane(e[g], j);
        bool mine_first = ranks_before(b[g], e[g], pb, pe);
        if (mine_first != keep_first) {
          b[g] = pb;
          e[g] = pe;
        }
      }
    }
  }
}

// a, c: sorted descending across the lanes.  Leaves the 64 first of a and c
// in a, sorted: the lane-wise better of a[i] and c[63 - i] is a bitonic
// sequence holding them, which a half-cleaner cascade sorts.
__device__ __forceinline__ void merge64(double& ab, int& ae, double cb, int ce, int lane) {
  double rb = xor_lane(cb, 63);
  int re = xor_lane(ce, 63);
  if (ranks_before(rb, re, ab, ae)) {
    ab = rb;
    ae = re;
  }
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) {
    double pb = xor_lane(ab, j);
    int pe = xor_lane(ae, j);
    const bool lower = (lane & j) == 0;
    if (ranks_before(ab, ae, pb, pe) != lower) {
      ab = pb;
      ae = pe;
    }
  }
}

// Exclusive prefix sum of arr[0, n) (n <= 4 * kThreads) in place; returns
// the total.  Called by all kThreads threads.
__device__ int block_scan(int* arr, int n, int* tmp4) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int v[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int i = tid * 4 + q;
    v[q] = i < n ? arr[i] : 0;
    sum += v[q];
  }
  int inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) tmp4[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += tmp4[w];
  int total = tmp4[0] + tmp4[1] + tmp4[2] + tmp4[3];
  int run = base + inc - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int i = tid * 4 + q;
    if (i < n) arr[i] = run;
    run += v[q];
  }
  __syncthreads();
  return total;
}

struct PlanLds {
  int ids[kMaxTokens * kMaxTopk];
  float w[kMaxTokens * kMaxTopk];
  int cnt[kMaxExperts];
  int base[kMaxExperts];
  int vsb[kMaxExperts];
  int tmp4[4];
  int last;
};

// Top-k of every token, its weights, then the plan.  Run by the last block.
template <int NG>
__device__ void route_and_plan(const LayerDims& d, int m, const float* __restrict__ bias, const Scratch& s,
                               PlanLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = d.E, K = d.K;

  for (int t = wave; t < m; t += kThreads / 64) {
    double b[NG];
    int e[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      int ex = 64 * g + lane;
      if (ex < E) {
        double l = __builtin_nontemporal_load(&s.logits[(size_t)t * E + ex]);
        double bb = 1.0 / (1.0 + exp(-l)) + (double)bias[ex];
        // a NaN score ranks last among the real experts, never below the
        // padding, so the picks are always real experts
        b[g] = (bb == bb) ? bb : -INFINITY;
        e[g] = ex;
      } else {
        b[g] = -INFINITY;
        e[g] = ex;  // distinct, above every real expert
      }
    }
    sort64<NG>(b, e, lane);
#pragma unroll
    for (int width = NG / 2; width >= 1; width >>= 1) {
#pragma unroll
      for (int g = 0; g < width; ++g) merge64(b[g], e[g], b[g + width], e[g + width], lane);
    }
    // lanes [0, K) hold the picks in selection order
    double sg = 0.0;
    if (lane < K) sg = 1.0 / (1.0 + exp(-__builtin_nontemporal_load(&s.logits[(size_t)t * E + e[0]])));
    double ssum = wave_sum(sg);
    if (lane < K) {
      float w = (float)((double)d.routed_scale * sg / ssum);
      s.ids[t * K + lane] = e[0];
      s.wts[t * K + lane] = w;
      L.ids[t * K + lane] = e[0];
      L.w[t * K + lane] = w;
    }
  }
  __syncthreads();

  // Tokens per expert, then rows (expert ascending, token ascending) and
  // virtual slots of at most kTokTile rows.
  const int P = m * K;
  for (int ex = tid; ex < E; ex += kThreads) {
    int c = 0;
    for (int p = 0; p < P; ++p) c += (L.ids[p] == ex);
    L.cnt[ex] = c;
    L.base[ex] = c;
    L.vsb[ex] = (c + kTokTile - 1) / kTokTile;
    s.counts[ex] = c;
  }
  __syncthreads();
  block_scan(L.base, E, L.tmp4);
  const int nR = block_scan(L.vsb, E, L.tmp4);
  const int nS = (m + kTokTile - 1) / kTokTile;
  for (int ex = tid; ex < E; ex += kThreads) {
    const int c = L.cnt[ex];
    if (c == 0) continue;
    int r = L.base[ex];
    for (int p = 0; p < P; ++p) {
      if (L.ids[p] == ex) {
        s.row_tok[r] = p / K;
        s.row_w[r] = L.w[p];
        s.pair_row[p] = r;
        ++r;
      }
    }
    for (int v = 0; v * kTokTile < c; ++v) {
      int rows = c - v * kTokTile;
      s.vslots[nS + L.vsb[ex] + v] = make_int4(ex, L.base[ex] + v * kTokTile, rows < kTokTile ? rows : kTokTile, 0);
    }
  }
  for (int t = tid; t < m; t += kThreads) {
    s.row_tok[P + t] = t;
    s.row_w[P + t] = 1.0f;
  }
  for (int v = tid; v < nS; v += kThreads) {
    int rows = m - v * kTokTile;
    s.vslots[v] = make_int4(-1, P + v * kTokTile, rows < kTokTile ? rows : kTokTile, 0);
  }
  if (tid == 0) {
    s.header[0] = nS + nR;
    s.header[1] = nS;
    s.header[2] = nS * (d.Is / 32) + nR * (d.I / 32);
    s.header[3] = m;
    __hip_atomic_store(s.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int EPB, int NG>
__global__ __launch_bounds__(kThreads) void seam_kernel(LayerDims d, int m, Inputs in, Scratch s) {
  __shared__ PlanLds L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blk = blockIdx.x, nblk = gridDim.x;
  const int H = d.H, E = d.E;
  const int e0 = blk * EPB;
  const int nchunk = (H + 511) / 512;  // 8 columns per lane per chunk

  for (int t = wave; t < m; t += kThreads / 64) {
    const uint16_t* xr = in.x + (size_t)t * H;
    // sum of squares in double: each square of a bf16 is exact
    double ss = 0.0;
    for (int it = 0; it < nchunk; ++it) {
      const int c = it * 512 + lane * 8;
      if (c < H) {
        u32x4 v = ld16(reinterpret_cast<const uint8_t*>(xr + c));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          double lo = bf16_to_f32(v[q] & 0xFFFFu), hi = bf16_to_f32(v[q] >> 16);
          ss += lo * lo;
          ss += hi * hi;
        }
      }
    }
    ss = wave_sum(ss);
    const float r = (float)(1.0 / sqrt(ss / (double)H + (double)d.eps));
    const bool owner = (t % nblk) == blk;

    double acc[EPB];
#pragma unroll
    for (int q = 0; q < EPB; ++q) acc[q] = 0.0;
    for (int it = 0; it < nchunk; ++it) {
      const int c = it * 512 + lane * 8;
      const bool live = c < H;
      float y[8];
      uint32_t yb[8];
      if (live) {
        u32x4 xv = ld16(reinterpret_cast<const uint8_t*>(xr + c));
        u32x4 wv = ld16(reinterpret_cast<const uint8_t*>(in.norm_w + c));
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          uint32_t xb = (q & 1) ? (xv[q >> 1] >> 16) : (xv[q >> 1] & 0xFFFFu);
          uint32_t wb = (q & 1) ? (wv[q >> 1] >> 16) : (wv[q >> 1] & 0xFFFFu);
          float xr_ = bf16_to_f32(xb) * r;   // fp32 product, rounded
          float yw = xr_ * bf16_to_f32(wb);  // fp32 product, rounded
          yb[q] = f32_to_bf16(yw);
          y[q] = bf16_to_f32(yb[q]);
        }
#pragma unroll
        for (int q = 0; q < EPB; ++q) {
          if (e0 + q < E) {
            u32x4 gv = ld16(reinterpret_cast<const uint8_t*>(in.gate_w + (size_t)(e0 + q) * H + c));
#pragma unroll
            for (int z = 0; z < 8; ++z) {
              uint32_t gb = (z & 1) ? (gv[z >> 1] >> 16) : (gv[z >> 1] & 0xFFFFu);
              acc[q] += (double)y[z] * (double)bf16_to_f32(gb);  // exact products
            }
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          y[q] = 0.0f;
          yb[q] = 0;
        }
      }
      if (owner) {
        // store_normed: the bf16 row; store_x8: MXFP8 of each 32 columns
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(y[q]));
        amax = group_max(amax, 4);  // lanes 4i..4i+3 hold one 32-group
        const int code = e8m0_code(amax);
        const float mul = mx_mul(code);
        if (live) {
          u32x4 nv;
#pragma unroll
          for (int q = 0; q < 4; ++q) nv[q] = yb[2 * q] | (yb[2 * q + 1] << 16);
          *reinterpret_cast<u32x4*>(s.normed + (size_t)t * H + c) = nv;
          u32x2 qv;
          qv[0] = fp8x4(y[0] * mul, y[1] * mul, y[2] * mul, y[3] * mul);
          qv[1] = fp8x4(y[4] * mul, y[5] * mul, y[6] * mul, y[7] * mul);
          *reinterpret_cast<u32x2*>(s.x8 + (size_t)t * H + c) = qv;
          if ((lane & 3) == 0) s.x8s[(size_t)t * (H / 32) + c / 32] = (uint8_t)code;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < EPB; ++q) {
      double tot = wave_sum(acc[q]);
      if (lane == 0 && e0 + q < E) s.logits[(size_t)t * E + e0 + q] = tot;
    }
  }

  // Arrival: publish this block's writes, count it, and let the last block
  // through to the routing.  Nothing waits.
  __threadfence();
  __syncthreads();
  if (tid == 0) L.last = (atomicAdd(s.counter, 1u) == (uint32_t)(nblk - 1));
  __syncthreads();
  if (!L.last) return;
  __threadfence();
  route_and_plan<NG>(d, m, in.bias, s, L);
}

template <int EPB>
hipError_t launch_seam_ng(const LayerDims& d, int m, const Inputs& in, const Scratch& s, hipStream_t st) {
  const int groups = (d.E + 63) / 64;
  const int nblk = (d.E + EPB - 1) / EPB;
  if (groups <= 1) hipLaunchKernelGGL((seam_kernel<EPB, 1>), dim3(nblk), dim3(kThreads), 0, st, d, m, in, s);
  else if (groups <= 2) hipLaunchKernelGGL((seam_kernel<EPB, 2>), dim3(nblk), dim3(kThreads), 0, st, d, m, in, s);
  else if (groups <= 4) hipLaunchKernelGGL((seam_kernel<EPB, 4>), dim3(nblk), dim3(kThreads), 0, st, d, m, in, s);
  else if (groups <= 8) hipLaunchKernelGGL((seam_kernel<EPB, 8>), dim3(nblk), dim3(kThreads), 0, st, d, m, in, s);
  else hipLaunchKernelGGL((seam_kernel<EPB, 16>), dim3(nblk), dim3(kThreads), 0, st, d, m, in, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_seam(const LayerDims& d, int m, const Inputs& in, const Scratch& s, hipStream_t st) {
  // one to four experts per block, at most 256 blocks
  if (d.E <= 256) return launch_seam_ng<1>(d, m, in, s, st);
  if (d.E <= 512) return launch_seam_ng<2>(d, m, in, s, st);
  return launch_seam_ng<4>(d, m, in, s, st);
}

}  // namespace moe
