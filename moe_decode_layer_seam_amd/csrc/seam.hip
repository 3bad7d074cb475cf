// seam.hip -- the FFN seam and the router, two launches:
//   seam:  RMSNorm -> bf16 normed rows -> MXFP8 (x8, x8s); router logits in
//          double precision.  Blocks tile (experts) x (token rows).
//   route: per token, sigmoid + bias -> top-k by bitonic sort networks on
//          64-bit selection keys over expert groups of 64 (the four waves of
//          a block sort groups in parallel, then merge) -> routing weights;
//          the last block to finish writes the token->expert plan.
//
// Pages: "vllm.models.deepseek_v41.amd.mono.layer" run_ffn (the seam's norm,
// then the MoE), store_normed (the normed row, bf16), store_x8 (MXFP8 of 8
// columns per lane, amax over the 4 lanes of a 32-group, code, multiply,
// E4M3 pack); "vllm.models.deepseek_v41.amd.mono.runner" MonoLayerWeights
// (gate_w bf16 [E, H], bias f32 [E], the e_score_correction_bias);
// build_mono_ffn (expert groups of 64 for the routing sort networks);
// "vllm.models.deepseek_v41.amd.mono.attention.device" atomic_add_dev
// (relaxed device-scope counters: no L2 write-back or invalidate).
#include "device.hpp"
#include "kernels.hpp"
#include "route.hpp"

namespace moe {
namespace {

// ===========================================================================
// seam: norm, MXFP8, logits
// ===========================================================================

// Block (es, ts): experts [EPB es, +EPB) and token rows [TB ts, +TB).  Every
// thread covers CPT chunks of 8 columns, the block kSeamChunk consecutive
// columns per chunk.  The norm weight and the gate rows are loaded once, up front,
// when they fit in registers (PRE); the token rows are held in registers
// between the sum of squares and the normed row.
// LOGITS false: the norm and MXFP8 only (one block column owns every row;
// logits_kernel computes the logits from the stored rows).
template <int EPB, int CPT, int TB, bool LOGITS>
__global__ __launch_bounds__(kSeamThreads) void seam_kernel(LayerDims d, int m, Inputs in, Scratch s) {
  __shared__ double red_ss[TB][kSeamWaves];
  __shared__ double red_lg[TB][EPB][kSeamWaves];
  constexpr bool PRE = LOGITS && EPB * CPT <= 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int es = blockIdx.x, nES = gridDim.x;
  const int t0 = blockIdx.y * TB;
  const int nt = m - t0 < TB ? m - t0 : TB;
  const int H = d.H, E = d.E;
  const int e0 = es * EPB;
  stamp(s.tl_seam, kTlPoints, 0);
  {
    // the fused expert launch's counters start every run at zero
    const uint32_t nthr = gridDim.x * gridDim.y * kSeamThreads;
    for (uint32_t w = (blockIdx.y * gridDim.x + blockIdx.x) * kSeamThreads + tid; w < (uint32_t)s.nsync; w += nthr)
      store_coherent(&s.sync[w], 0u);
  }

  int col[CPT];
  bool live[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    col[q] = 8 * tid + kSeamChunk * q;
    live[q] = col[q] < H;
  }
  // the token rows first: loads complete in issue order, so the sum of
  // squares need not wait for the gate rows
  u32x4 xv[TB][CPT];
#pragma unroll
  for (int tt = 0; tt < TB; ++tt)
#pragma unroll
    for (int q = 0; q < CPT; ++q)
      if (tt < nt && live[q]) xv[tt][q] = ld16(reinterpret_cast<const uint8_t*>(in.x + (size_t)(t0 + tt) * H + col[q]));
  u32x4 wv[PRE ? CPT : 1], gv[PRE ? EPB : 1][PRE ? CPT : 1];
  if constexpr (PRE) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      if (live[q]) {
        wv[q] = ld16(reinterpret_cast<const uint8_t*>(in.norm_w + col[q]));
#pragma unroll
        for (int e = 0; e < EPB; ++e)
          if (e0 + e < E) gv[e][q] = ld16(reinterpret_cast<const uint8_t*>(in.gate_w + (size_t)(e0 + e) * H + col[q]));
      }
    }
  }

  // sum of squares in double: each square of a bf16 is exact; lanes, then
  // waves, are added in a fixed order
#pragma unroll
  for (int tt = 0; tt < TB; ++tt) {
    double ss = 0.0;
#pragma unroll
    for (int q = 0; q < CPT; ++q)
      if (tt < nt && live[q]) ss = add_squares8(ss, xv[tt][q]);
    ss = wave_sum(ss);
    if (lane == 0) red_ss[tt][wave] = ss;
  }
  __syncthreads();
  stamp(s.tl_seam, kTlPoints, 1);

#pragma unroll
  for (int tt = 0; tt < TB; ++tt) {
    if (tt >= nt) break;
    const int t = t0 + tt;
    double ss = red_ss[tt][0];
#pragma unroll
    for (int w = 1; w < kSeamWaves; ++w) ss += red_ss[tt][w];
    const float r = (float)(1.0 / sqrt(ss / (double)H + (double)d.eps));
    const bool owner = (t % nES) == es;
    double acc[EPB];
#pragma unroll
    for (int e = 0; e < EPB; ++e) acc[e] = 0.0;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      float y[8];
      uint32_t yb[8];
      if (live[q]) {
        u32x4 w;
        if constexpr (PRE) w = wv[q];
        else w = ld16(reinterpret_cast<const uint8_t*>(in.norm_w + col[q]));
        norm8(xv[tt][q], w, r, y, yb);
#pragma unroll
        for (int e = 0; e < EPB; ++e) {
          if (LOGITS && e0 + e < E) {
            u32x4 g;
            if constexpr (PRE) g = gv[e][q];
            else g = ld16(reinterpret_cast<const uint8_t*>(in.gate_w + (size_t)(e0 + e) * H + col[q]));
            acc[e] = add_logit8(acc[e], y, g);
          }
        }
      } else {
#pragma unroll
        for (int z = 0; z < 8; ++z) {
          y[z] = 0.0f;
          yb[z] = 0;
        }
      }
      if (owner) {
        // store_normed: the bf16 row; store_x8: MXFP8 of each 32 columns,
        // held by 4 consecutive lanes
        u32x2 qv;
        const int code = mx8(y, qv);
        if (live[q]) {
          u32x4 nv;
#pragma unroll
          for (int z = 0; z < 4; ++z) nv[z] = yb[2 * z] | (yb[2 * z + 1] << 16);
          *reinterpret_cast<u32x4*>(s.normed + (size_t)t * H + col[q]) = nv;
          *reinterpret_cast<u32x2*>(s.x8 + (size_t)t * H + col[q]) = qv;
          if ((lane & 3) == 0) s.x8s[(size_t)t * (H / 32) + col[q] / 32] = (uint8_t)code;
        }
      }
    }
    if (LOGITS) {
#pragma unroll
      for (int e = 0; e < EPB; ++e) {
        const double tot = wave_sum(acc[e]);
        if (lane == 0) red_lg[tt][e][wave] = tot;
      }
    }
  }
  if (!LOGITS) {
    stamp(s.tl_seam, kTlPoints, 2);
    return;
  }
  __syncthreads();
  for (int i = tid; i < nt * EPB; i += kSeamThreads) {
    const int tt = i / EPB, e = i % EPB;
    if (e0 + e < E) {
      double v = red_lg[tt][e][0];
#pragma unroll
      for (int w = 1; w < kSeamWaves; ++w) v += red_lg[tt][e][w];
      s.logits[(size_t)(t0 + tt) * E + e0 + e] = v;
    }
  }
  stamp(s.tl_seam, kTlPoints, 2);
}

// Rows per block: a block holds TB rows of CPT chunks in registers.
template <int CPT>
constexpr int seam_tb() {
  return CPT <= 2 ? 8 : 4;
}

// Router logits from the stored bf16 rows: block (es, ts) takes experts
// [EPB es, +EPB) and rows [TB ts, +TB).  Every logit is summed exactly as in
// seam_kernel (a thread's columns in the same order, the same wave sum, the
// waves in order), so both paths give the same bits.
template <int EPB, int CPT, int TB, bool ROUTE>
__global__ __launch_bounds__(kSeamThreads) void logits_kernel(LayerDims d, int m, Inputs in, Scratch s) {
  __shared__ double red_lg[TB][EPB][kSeamWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.y * TB;
  const int nt = m - t0 < TB ? m - t0 : TB;
  const int H = d.H, E = d.E;
  const int e0 = blockIdx.x * EPB;
  stamp(s.tl_logits, kTlPoints, 0);
  int col[CPT];
  bool live[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    col[q] = 8 * tid + kSeamChunk * q;
    live[q] = col[q] < H;
  }
  u32x4 yv[TB][CPT], gv[EPB][CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
#pragma unroll
    for (int tt = 0; tt < TB; ++tt)
      yv[tt][q] = (tt < nt && live[q]) ? ld16(reinterpret_cast<const uint8_t*>(s.normed + (size_t)(t0 + tt) * H + col[q]))
                                       : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < EPB; ++e)
      gv[e][q] = (e0 + e < E && live[q]) ? ld16(reinterpret_cast<const uint8_t*>(in.gate_w + (size_t)(e0 + e) * H + col[q]))
                                         : u32x4{0u, 0u, 0u, 0u};
  }
  double acc[TB][EPB];
#pragma unroll
  for (int tt = 0; tt < TB; ++tt)
#pragma unroll
    for (int e = 0; e < EPB; ++e) acc[tt][e] = 0.0;
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    if (!live[q]) continue;
#pragma unroll
    for (int z = 0; z < 8; ++z) {
      double yd[TB];
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        const uint32_t yb = (z & 1) ? (yv[tt][q][z >> 1] >> 16) : (yv[tt][q][z >> 1] & 0xFFFFu);
        yd[tt] = (double)bf16_to_f32(yb);
      }
#pragma unroll
      for (int e = 0; e < EPB; ++e) {
        const uint32_t gb = (z & 1) ? (gv[e][q][z >> 1] >> 16) : (gv[e][q][z >> 1] & 0xFFFFu);
        const double gd = (double)bf16_to_f32(gb);
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) acc[tt][e] += yd[tt] * gd;  // exact products
      }
    }
  }
  // every (row, expert) sum over the wave at once; lane l ends with value
  // l >> shift, value i = tt * EPB + e
  constexpr int NV = TB * EPB;
  constexpr int shift = NV >= 32 ? 1 : NV >= 16 ? 2 : NV >= 8 ? 3 : NV >= 4 ? 4 : NV >= 2 ? 5 : 6;
  double v[NV];
#pragma unroll
  for (int tt = 0; tt < TB; ++tt)
#pragma unroll
    for (int e = 0; e < EPB; ++e) v[tt * EPB + e] = acc[tt][e];
  reduce_scatter<NV>(v, lane);
  if ((lane & ((1 << shift) - 1)) == 0) {
    const int i = lane >> shift;
    red_lg[i / EPB][i % EPB][wave] = v[0];
  }
  __syncthreads();
  for (int i = tid; i < nt * EPB; i += kSeamThreads) {
    const int tt = i / EPB, e = i % EPB;
    if (e0 + e < E) {
      double v = red_lg[tt][e][0];
#pragma unroll
      for (int w = 1; w < kSeamWaves; ++w) v += red_lg[tt][e][w];
      if constexpr (ROUTE)  // read by the tile's last block: stored through
        __hip_atomic_store(reinterpret_cast<uint64_t*>(s.logits) + (size_t)(t0 + tt) * E + e0 + e,
                           (uint64_t)__double_as_longlong(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        s.logits[(size_t)(t0 + tt) * E + e0 + e] = v;
    }
  }
  if constexpr (ROUTE) {
    // the tile's last block to arrive (its blocks' logits stored and
    // completed before each counts itself) routes the tile's rows, one wave
    // a row; it then zeroes the count for the next step
    __shared__ int s_last;
    wait_memory();
    __syncthreads();
    if (tid == 0) {
      uint32_t* cnt = s.tile_cnt + (size_t)blockIdx.y * kTileCntStride;
      s_last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1u;
    }
    __syncthreads();
    if (s_last) {
      if (wave < nt) route_wave(d, t0 + wave, in.bias, s, lane);
      if (tid == 0) __hip_atomic_store(s.tile_cnt + (size_t)blockIdx.y * kTileCntStride, 0u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  stamp(s.tl_logits, kTlPoints, 1);
}

template <int EPB, int CPT, bool LOGITS>
hipError_t launch_seam_t(const LayerDims& d, int m, const Inputs& in, const Scratch& s, hipStream_t st,
                         const KernelEvents& ev) {
  constexpr int TB = LOGITS ? seam_tb<CPT>() : 1;
  const dim3 grid(LOGITS ? (d.E + EPB - 1) / EPB : 1, (m + TB - 1) / TB);
  return launch_kernel(seam_kernel<EPB, CPT, TB, LOGITS>, grid, dim3(kSeamThreads), 0, st, ev, d, m, in, s);
}

template <int EPB, bool LOGITS>
hipError_t launch_seam_epb(const LayerDims& d, int m, const Inputs& in, const Scratch& s, hipStream_t st,
                           const KernelEvents& ev) {
  switch (seam_cpt(d.H)) {
    case 1: return launch_seam_t<EPB, 1, LOGITS>(d, m, in, s, st, ev);
    case 2: return launch_seam_t<EPB, 2, LOGITS>(d, m, in, s, st, ev);
    case 3: return launch_seam_t<EPB, 3, LOGITS>(d, m, in, s, st, ev);
    default: return launch_seam_t<EPB, 4, LOGITS>(d, m, in, s, st, ev);
  }
}

// Logits tiles: 4 rows x 4 experts when a thread's chunks of the row number
// at most 2 (registers), else 4 rows x 2 experts.  At H = 5120, E = 256 this
// takes 9.5 us at m = 48 and 4.5 us at m = 16; tiles of 8 x 4, 4 x 8 or
// 8 x 2 took 12 and 4.7-6.3 us.  A logit is summed in the same tree
// whatever the tile.
// route: the launch also routes the rows (one sort group, E <= 64).
template <int CPT>
hipError_t launch_logits_t(const LayerDims& d, int m, const Inputs& in, const Scratch& s, bool route, hipStream_t st,
                           const KernelEvents& ev) {
  constexpr int TB = 4, EPB = CPT <= 2 ? 4 : 2;
  const dim3 grid((d.E + EPB - 1) / EPB, (m + TB - 1) / TB);
  if (route)
    return launch_kernel(logits_kernel<EPB, CPT, TB, true>, grid, dim3(kSeamThreads), 0, st, ev, d, m, in, s);
  return launch_kernel(logits_kernel<EPB, CPT, TB, false>, grid, dim3(kSeamThreads), 0, st, ev, d, m, in, s);
}

// ===========================================================================
// route: top-k per token, weights, plan (route.hpp)
// ===========================================================================

template <int GPW>
__global__ __launch_bounds__(kThreads) void route_kernel(LayerDims d, int m, const float* __restrict__ bias,
                                                         Scratch s, int plan) {
  __shared__ RouteLds L;
  (void)route_block<GPW>(d, m, blockIdx.x, gridDim.x, bias, s, L, nullptr, nullptr, plan != 0);
}

}  // namespace

hipError_t launch_seam(const LayerDims& d, int m, const Inputs& in, const Scratch& s, hipStream_t st,
                       const KernelEvents& ev) {
  if (!seam_fused(m)) return launch_seam_epb<1, false>(d, m, in, s, st, ev);
  const int epb = seam_epb(d, m);
  if (epb == 1) return launch_seam_epb<1, true>(d, m, in, s, st, ev);
  if (epb == 2) return launch_seam_epb<2, true>(d, m, in, s, st, ev);
  if (epb == 4) return launch_seam_epb<4, true>(d, m, in, s, st, ev);
  return launch_seam_epb<8, true>(d, m, in, s, st, ev);
}

hipError_t launch_logits(const LayerDims& d, int m, const Inputs& in, const Scratch& s, bool route, hipStream_t st,
                         const KernelEvents& ev) {
  switch (seam_cpt(d.H)) {
    case 1: return launch_logits_t<1>(d, m, in, s, route, st, ev);
    case 2: return launch_logits_t<2>(d, m, in, s, route, st, ev);
    case 3: return launch_logits_t<3>(d, m, in, s, route, st, ev);
    default: return launch_logits_t<4>(d, m, in, s, route, st, ev);
  }
}

hipError_t launch_route(const LayerDims& d, int m, const Inputs& in, const Scratch& s, bool plan, hipStream_t st,
                        const KernelEvents& ev) {
  const int groups = (d.E + 63) / 64;  // sort groups; wave w takes w, w+4, ...
  const int gpw = (groups + 3) / 4;
  const int pl = plan ? 1 : 0;
  if (gpw <= 1) return launch_kernel(route_kernel<1>, dim3(m), dim3(kThreads), 0, st, ev, d, m, in.bias, s, pl);
  if (gpw <= 2) return launch_kernel(route_kernel<2>, dim3(m), dim3(kThreads), 0, st, ev, d, m, in.bias, s, pl);
  return launch_kernel(route_kernel<4>, dim3(m), dim3(kThreads), 0, st, ev, d, m, in.bias, s, pl);
}

}  // namespace moe
