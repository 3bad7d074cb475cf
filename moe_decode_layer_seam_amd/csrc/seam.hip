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

namespace moe {
namespace {

// ===========================================================================
// seam: norm, MXFP8, logits
// ===========================================================================

// Block (es, ts): experts [EPB es, +EPB) and token rows [TB ts, +TB).  Every
// thread covers CPT chunks of 8 columns, the block 2048 consecutive columns
// per chunk.  The norm weight and the gate rows are loaded once, up front,
// when they fit in registers (PRE); the token rows are held in registers
// between the sum of squares and the normed row.
// LOGITS false: the norm and MXFP8 only (one block column owns every row;
// logits_kernel computes the logits from the stored rows).
template <int EPB, int CPT, int TB, bool LOGITS>
__global__ __launch_bounds__(kThreads) void seam_kernel(LayerDims d, int m, Inputs in, Scratch s) {
  __shared__ double red_ss[TB][4];
  __shared__ double red_lg[TB][EPB][4];
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
    const uint32_t nthr = gridDim.x * gridDim.y * kThreads;
    for (uint32_t w = (blockIdx.y * gridDim.x + blockIdx.x) * kThreads + tid; w < (uint32_t)s.nsync; w += nthr)
      store_coherent(&s.sync[w], 0u);
  }

  int col[CPT];
  bool live[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    col[q] = 8 * tid + 2048 * q;
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
    for (int q = 0; q < CPT; ++q) {
      if (tt < nt && live[q]) {
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          const double lo = bf16_to_f32(xv[tt][q][z] & 0xFFFFu), hi = bf16_to_f32(xv[tt][q][z] >> 16);
          ss += lo * lo;
          ss += hi * hi;
        }
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red_ss[tt][wave] = ss;
  }
  __syncthreads();
  stamp(s.tl_seam, kTlPoints, 1);

#pragma unroll
  for (int tt = 0; tt < TB; ++tt) {
    if (tt >= nt) break;
    const int t = t0 + tt;
    const double ss = red_ss[tt][0] + red_ss[tt][1] + red_ss[tt][2] + red_ss[tt][3];
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
#pragma unroll
        for (int z = 0; z < 8; ++z) {
          const uint32_t xb = (z & 1) ? (xv[tt][q][z >> 1] >> 16) : (xv[tt][q][z >> 1] & 0xFFFFu);
          const uint32_t wb = (z & 1) ? (w[z >> 1] >> 16) : (w[z >> 1] & 0xFFFFu);
          const float xr = bf16_to_f32(xb) * r;   // fp32 product, rounded
          const float yw = xr * bf16_to_f32(wb);  // fp32 product, rounded
          yb[z] = f32_to_bf16(yw);
          y[z] = bf16_to_f32(yb[z]);
        }
#pragma unroll
        for (int e = 0; e < EPB; ++e) {
          if (LOGITS && e0 + e < E) {
            u32x4 g;
            if constexpr (PRE) g = gv[e][q];
            else g = ld16(reinterpret_cast<const uint8_t*>(in.gate_w + (size_t)(e0 + e) * H + col[q]));
#pragma unroll
            for (int z = 0; z < 8; ++z) {
              const uint32_t gb = (z & 1) ? (g[z >> 1] >> 16) : (g[z >> 1] & 0xFFFFu);
              acc[e] += (double)y[z] * (double)bf16_to_f32(gb);  // exact products
            }
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
        float amax = 0.0f;
#pragma unroll
        for (int z = 0; z < 8; ++z) amax = fmaxf(amax, fabsf(y[z]));
        amax = group_max(amax, 4);
        const int code = e8m0_code(amax);
        const float mul = mx_mul(code);
        if (live[q]) {
          u32x4 nv;
#pragma unroll
          for (int z = 0; z < 4; ++z) nv[z] = yb[2 * z] | (yb[2 * z + 1] << 16);
          *reinterpret_cast<u32x4*>(s.normed + (size_t)t * H + col[q]) = nv;
          u32x2 qv;
          qv[0] = fp8x4(y[0] * mul, y[1] * mul, y[2] * mul, y[3] * mul);
          qv[1] = fp8x4(y[4] * mul, y[5] * mul, y[6] * mul, y[7] * mul);
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
  for (int i = tid; i < nt * EPB; i += kThreads) {
    const int tt = i / EPB, e = i % EPB;
    if (e0 + e < E)
      s.logits[(size_t)(t0 + tt) * E + e0 + e] = red_lg[tt][e][0] + red_lg[tt][e][1] + red_lg[tt][e][2] + red_lg[tt][e][3];
  }
  stamp(s.tl_seam, kTlPoints, 2);
}

// Rows per block: a block holds TB rows of CPT chunks in registers.
template <int CPT>
constexpr int seam_tb() {
  return CPT <= 4 ? 8 : 4;
}

// Router logits from the stored bf16 rows: block (es, ts) takes experts
// [EPB es, +EPB) and rows [TB ts, +TB).  Every logit is summed exactly as in
// seam_kernel (a thread's columns in the same order, the same wave sum, the
// four waves in order), so both paths give the same bits.
template <int EPB, int CPT, int TB>
__global__ __launch_bounds__(kThreads) void logits_kernel(LayerDims d, int m, Inputs in, Scratch s) {
  __shared__ double red_lg[TB][EPB][4];
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
    col[q] = 8 * tid + 2048 * q;
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
  for (int i = tid; i < nt * EPB; i += kThreads) {
    const int tt = i / EPB, e = i % EPB;
    if (e0 + e < E)
      s.logits[(size_t)(t0 + tt) * E + e0 + e] = red_lg[tt][e][0] + red_lg[tt][e][1] + red_lg[tt][e][2] + red_lg[tt][e][3];
  }
  stamp(s.tl_logits, kTlPoints, 1);
}

template <int EPB, int CPT, bool LOGITS>
hipError_t launch_seam_t(const LayerDims& d, int m, const Inputs& in, const Scratch& s, hipStream_t st,
                         const KernelEvents& ev) {
  constexpr int TB = LOGITS ? seam_tb<CPT>() : 1;
  const dim3 grid(LOGITS ? (d.E + EPB - 1) / EPB : 1, (m + TB - 1) / TB);
  return launch_kernel(seam_kernel<EPB, CPT, TB, LOGITS>, grid, dim3(kThreads), 0, st, ev, d, m, in, s);
}

template <int EPB, bool LOGITS>
hipError_t launch_seam_epb(const LayerDims& d, int m, const Inputs& in, const Scratch& s, hipStream_t st,
                           const KernelEvents& ev) {
  switch ((d.H + 2047) / 2048) {
    case 1: return launch_seam_t<EPB, 1, LOGITS>(d, m, in, s, st, ev);
    case 2: return launch_seam_t<EPB, 2, LOGITS>(d, m, in, s, st, ev);
    case 3: return launch_seam_t<EPB, 3, LOGITS>(d, m, in, s, st, ev);
    case 4: return launch_seam_t<EPB, 4, LOGITS>(d, m, in, s, st, ev);
    case 5: return launch_seam_t<EPB, 5, LOGITS>(d, m, in, s, st, ev);
    case 6: return launch_seam_t<EPB, 6, LOGITS>(d, m, in, s, st, ev);
    case 7: return launch_seam_t<EPB, 7, LOGITS>(d, m, in, s, st, ev);
    default: return launch_seam_t<EPB, 8, LOGITS>(d, m, in, s, st, ev);
  }
}

// Logits tiles: 4 experts x 4 rows when the row is up to 2048 columns per
// thread chunk budget allows it (registers), else 2 x 4.
template <int CPT>
hipError_t launch_logits_t(const LayerDims& d, int m, const Inputs& in, const Scratch& s, hipStream_t st,
                           const KernelEvents& ev) {
  constexpr int TB = CPT <= 3 ? 8 : 4, EPB = CPT <= 3 ? 4 : 2;
  const dim3 grid((d.E + EPB - 1) / EPB, (m + TB - 1) / TB);
  return launch_kernel(logits_kernel<EPB, CPT, TB>, grid, dim3(kThreads), 0, st, ev, d, m, in, s);
}

// ===========================================================================
// route: top-k per token, weights, plan
// ===========================================================================

// Exclusive prefix sum of arr[0, n) (n <= 4 * kThreads) in place; returns
// the total.  Called by all kThreads threads.
__device__ int block_scan(int* arr, int n, int* tmp4) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int v[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = tid * 4 + q;
    v[q] = i < n ? arr[i] : 0;
    sum += v[q];
  }
  int inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) tmp4[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += tmp4[w];
  const int total = tmp4[0] + tmp4[1] + tmp4[2] + tmp4[3];
  int run = base + inc - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = tid * 4 + q;
    if (i < n) arr[i] = run;
    run += v[q];
  }
  __syncthreads();
  return total;
}

struct RouteLds {
  uint64_t cand[4][64];      // each wave's sorted selection keys
  double sig[kMaxExperts];   // this token's sigmoid scores
  int ids[kMaxTokens * kMaxTopk];
  float w[kMaxTokens * kMaxTopk];
  uint32_t mlo[kMaxExperts], mhi[kMaxExperts];  // tokens 0-31 / 32-47 per expert
  int base[kMaxExperts];
  int vsb[kMaxExperts];
  int tmp4[4];
  int last;
};

// The plan of a step of at most 64 pairs and 16 tokens, by wave 0 alone:
// lane p takes pair p, a bitonic sort of the keys expert * 64 + token puts
// row r's pair in lane r, and every expert has one virtual slot (its rows
// are at most the 16 tokens).  Same plan as build_plan's general path.
__device__ void plan_small(const LayerDims& d, int m, const Scratch& s, RouteLds& L, int lane) {
  const int E = d.E, K = d.K, P = m * K;
  // key: expert, token, pair (10 + 4 + 6 bits), unique; sorted ascending over
  // the smallest power-of-two number of lanes that holds the pairs
  int key = 0x7FFFFFFF;
  if (lane < P) key = (L.ids[lane] << 10) | ((lane / K) << 6) | lane;
  const int width = P <= 8 ? 8 : (P <= 16 ? 16 : (P <= 32 ? 32 : 64));
  // (every stage unrolled, so each exchange is a fixed DPP or permlane
  // pattern; a level is skipped as a whole when it is wider than needed)
#pragma unroll
  for (int k2 = 2; k2 <= 64; k2 <<= 1) {
    if (k2 <= width) {
#pragma unroll
      for (int j = k2 >> 1; j > 0; j >>= 1) {
        const int pk = xor_lane(key, j);
        // ascending: the lower lane of a pair keeps the smaller key when up
        const bool keep_min = ((lane & j) == 0) == ((lane & k2) == 0);
        key = keep_min ? min(key, pk) : max(key, pk);
      }
    }
  }
  const int r = lane;
  const bool valid = r < P;
  const int e = key >> 10, t = (key >> 6) & 15, p = key & 63;
  const int eprev = __shfl_up(e, 1, 64);
  const bool first = valid && (r == 0 || eprev != e);
  const uint64_t fm = __ballot(first);
  const uint64_t above = r == 63 ? 0ull : fm & ~((2ull << r) - 1ull);
  const int cnt = (above ? __ffsll((unsigned long long)above) - 1 : P) - r;
  const int nR = __popcll(fm), nS = 1;
  if (valid) {
    s.row_tok[r] = t;
    s.row_w[r] = L.w[p];
    s.pair_row[p] = r;
    s.row_out[r] = p;
  }
  if (first) s.vslots[nS + __popcll(fm & ((1ull << r) - 1ull))] = make_int4(e, r, cnt, 0);
  // tokens per expert: a table in LDS (one wave: its LDS accesses are in
  // order), then copied out whole
  for (int x = lane; x < E; x += 64) L.base[x] = 0;
  if (first) L.base[e] = cnt;
  for (int x = lane; x < E; x += 64) s.counts[x] = L.base[x];
  if (lane < m) {
    s.row_tok[P + lane] = lane;
    s.row_w[P + lane] = 1.0f;
    s.row_out[P + lane] = P + lane;
  }
  if (lane == 0) {
    s.vslots[0] = make_int4(-1, P, m, 0);
    s.header[0] = nS + nR;
    s.header[1] = nS;
    s.header[2] = nR;
    s.header[3] = m;
    __hip_atomic_store(s.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The plan, from every token's picks: rows listed by expert ascending, then
// token ascending; an expert's rows split into virtual slots of at most
// kTokTile rows; the shared expert's m rows last, its slots first.  With at
// most 48 tokens, the tokens of an expert form one 64-bit mask and a pair's
// rank within its expert is the count of lower tokens in the mask.
// own: the token whose picks this block holds in LDS already.
__device__ void build_plan(const LayerDims& d, int m, int own, const Scratch& s, RouteLds& L) {
  const int tid = threadIdx.x;
  const int E = d.E, K = d.K, P = m * K;
  for (int p = tid; p < P; p += kThreads) {
    if (p / K == own) continue;
    L.ids[p] = __hip_atomic_load(&s.ids[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    L.w[p] = __hip_atomic_load(&s.wts[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (P <= 64 && m <= kTokTile) {
    __syncthreads();
    if (threadIdx.x < 64) plan_small(d, m, s, L, threadIdx.x);
    return;
  }
  for (int e = tid; e < E; e += kThreads) L.mlo[e] = L.mhi[e] = 0u;
  __syncthreads();
  for (int p = tid; p < P; p += kThreads) {
    const int t = p / K, e = L.ids[p];
    if (t < 32) atomicOr(&L.mlo[e], 1u << t);
    else atomicOr(&L.mhi[e], 1u << (t - 32));
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    const int c = __popc(L.mlo[e]) + __popc(L.mhi[e]);
    L.base[e] = c;
    L.vsb[e] = (c + kTokTile - 1) / kTokTile;
    s.counts[e] = c;
  }
  __syncthreads();
  block_scan(L.base, E, L.tmp4);
  const int nR = block_scan(L.vsb, E, L.tmp4);
  const int nS = (m + kTokTile - 1) / kTokTile;
  for (int p = tid; p < P; p += kThreads) {
    const int t = p / K, e = L.ids[p];
    const int rank = t < 32 ? __popc(L.mlo[e] & ((1u << t) - 1u))
                            : __popc(L.mlo[e]) + __popc(L.mhi[e] & ((1u << (t - 32)) - 1u));
    const int r = L.base[e] + rank;
    s.row_tok[r] = t;
    s.row_w[r] = L.w[p];
    s.pair_row[p] = r;
    s.row_out[r] = p;
  }
  for (int e = tid; e < E; e += kThreads) {
    const int c = __popc(L.mlo[e]) + __popc(L.mhi[e]);
    for (int v = 0; v * kTokTile < c; ++v) {
      const int rows = c - v * kTokTile;
      s.vslots[nS + L.vsb[e] + v] = make_int4(e, L.base[e] + v * kTokTile, rows < kTokTile ? rows : kTokTile, 0);
    }
  }
  for (int t = tid; t < m; t += kThreads) {
    s.row_tok[P + t] = t;
    s.row_w[P + t] = 1.0f;
    s.row_out[P + t] = P + t;
  }
  for (int v = tid; v < nS; v += kThreads) {
    const int rows = m - v * kTokTile;
    s.vslots[v] = make_int4(-1, P + v * kTokTile, rows < kTokTile ? rows : kTokTile, 0);
  }
  if (tid == 0) {
    s.header[0] = nS + nR;
    s.header[1] = nS;
    s.header[2] = nR;
    s.header[3] = m;
    __hip_atomic_store(s.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Selection key of expert e with biased score b: the fp64 order of b
// (larger first) in the upper 54 bits, then the lower index first.  Scores
// closer than 2^-42 relative (below the 10 low bits) fall to the index.
__device__ __forceinline__ uint64_t select_key(double b, int e) {
  const uint64_t u = (uint64_t)__double_as_longlong(b + 0.0);  // -0 -> +0
  const uint64_t mono = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
  return (mono & ~0x3FFull) | (uint64_t)(1023 - e);
}

__device__ __forceinline__ uint64_t xor_lane64(uint64_t v, int mask) {
  const int lo = xor_lane((int)(uint32_t)v, mask), hi = xor_lane((int)(uint32_t)(v >> 32), mask);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Bitonic sorting network over the 64 lanes, descending, on G independent
// lists at once.
template <int G>
__device__ __forceinline__ void sort64(uint64_t (&k)[G], int lane) {
#pragma unroll
  for (int k2 = 2; k2 <= 64; k2 <<= 1) {
#pragma unroll
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      const bool keep_max = ((lane & j) == 0) == ((lane & k2) == 0);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint64_t p = xor_lane64(k[g], j);
        k[g] = keep_max ? (p > k[g] ? p : k[g]) : (p < k[g] ? p : k[g]);
      }
    }
  }
}

// a, c: sorted descending across the lanes.  Leaves the 64 largest of both
// in a, sorted: the lane-wise larger of a[i] and c[63 - i] is a bitonic
// sequence holding them, which a half-cleaner cascade sorts.
__device__ __forceinline__ void merge64(uint64_t& a, uint64_t c, int lane) {
  const uint64_t r = xor_lane64(c, 63);
  a = r > a ? r : a;
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) {
    const uint64_t p = xor_lane64(a, j);
    a = ((lane & j) == 0) ? (p > a ? p : a) : (p < a ? p : a);
  }
}

// Block t: token t.  Wave w sorts the selection keys of expert groups w,
// w + 4, ... (GPW groups of 64) and merges them; wave 0 merges the four
// waves' lists, and its lanes [0, k) hold the picks in selection order.
template <int GPW>
__global__ __launch_bounds__(kThreads) void route_kernel(LayerDims d, int m, const float* __restrict__ bias,
                                                         Scratch s) {
  __shared__ RouteLds L;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = blockIdx.x;
  const int E = d.E, K = d.K;
  const int groups = (E + 63) / 64;
  stamp(s.tl_route, kTlPoints, 0);

  uint64_t k[GPW];
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    const int ex = 64 * (wave + 4 * i) + lane;
    k[i] = 0;  // below every real expert's key
    if (ex < E) {
      const double sg = 1.0 / (1.0 + exp(-s.logits[(size_t)t * E + ex]));
      const double bb = sg + (double)bias[ex];
      L.sig[ex] = sg;
      k[i] = select_key((bb == bb) ? bb : -INFINITY, ex);  // a NaN score ranks last
    }
  }
  stamp(s.tl_route, kTlPoints, 5);
  if (wave < groups) {
    sort64<GPW>(k, lane);
#pragma unroll
    for (int width = GPW / 2; width >= 1; width >>= 1) {
#pragma unroll
      for (int i = 0; i < width; ++i) merge64(k[i], k[i + width], lane);
    }
  }
  L.cand[wave][lane] = k[0];
  __syncthreads();
  stamp(s.tl_route, kTlPoints, 1);
  if (wave == 0) {
    const int nw = groups < 4 ? groups : 4;
    if (K <= 16) {
      // the four lists' top 16 side by side (lanes [16 w, +16)), merged by
      // two bitonic merges: pairs of 16 into 32, then 32 into 64
      k[0] = (lane >> 4) < nw ? L.cand[lane >> 4][lane & 15] : 0ull;
      uint64_t p = xor_lane64(k[0], 31);
      k[0] = (lane & 16) == 0 ? (p > k[0] ? p : k[0]) : (p < k[0] ? p : k[0]);
#pragma unroll
      for (int j = 8; j > 0; j >>= 1) {
        p = xor_lane64(k[0], j);
        k[0] = (lane & j) == 0 ? (p > k[0] ? p : k[0]) : (p < k[0] ? p : k[0]);
      }
      p = xor_lane64(k[0], 63);
      k[0] = (lane & 32) == 0 ? (p > k[0] ? p : k[0]) : (p < k[0] ? p : k[0]);
#pragma unroll
      for (int j = 16; j > 0; j >>= 1) {
        p = xor_lane64(k[0], j);
        k[0] = (lane & j) == 0 ? (p > k[0] ? p : k[0]) : (p < k[0] ? p : k[0]);
      }
    } else {
      for (int w = 1; w < nw; ++w) merge64(k[0], L.cand[w][lane], lane);
    }
    stamp(s.tl_route, kTlPoints, 6);
    const int e = 1023 - (int)(k[0] & 0x3FF);
    const double sg = lane < K ? L.sig[e] : 0.0;
    const double ssum = wave_sum(sg);
    if (lane < K) {
      const float w = (float)((double)d.routed_scale * sg / ssum);
      L.ids[t * K + lane] = e;
      L.w[t * K + lane] = w;
      // read by another block of this launch: stored device-coherent
      __hip_atomic_store(&s.ids[t * K + lane], e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&s.wts[t * K + lane], w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  stamp(s.tl_route, kTlPoints, 2);

  if (gridDim.x > 1) {
    // Arrival: wait until this block's coherent stores completed, count the
    // block, and let the last one through to the plan.  Nothing spins.  (A
    // workgroup-scope fence would not wait for the stores: only the explicit
    // wait orders them before the count.)
    wait_memory();
    __syncthreads();
    if (tid == 0)
      L.last = (__hip_atomic_fetch_add(s.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)(gridDim.x - 1));
    __syncthreads();
    if (!L.last) return;
  } else {
    __syncthreads();
  }
  stamp(s.tl_route, kTlPoints, 3);
  build_plan(d, m, t, s, L);
  stamp(s.tl_route, kTlPoints, 4);
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

hipError_t launch_logits(const LayerDims& d, int m, const Inputs& in, const Scratch& s, hipStream_t st,
                         const KernelEvents& ev) {
  switch ((d.H + 2047) / 2048) {
    case 1: return launch_logits_t<1>(d, m, in, s, st, ev);
    case 2: return launch_logits_t<2>(d, m, in, s, st, ev);
    case 3: return launch_logits_t<3>(d, m, in, s, st, ev);
    case 4: return launch_logits_t<4>(d, m, in, s, st, ev);
    case 5: return launch_logits_t<5>(d, m, in, s, st, ev);
    case 6: return launch_logits_t<6>(d, m, in, s, st, ev);
    case 7: return launch_logits_t<7>(d, m, in, s, st, ev);
    default: return launch_logits_t<8>(d, m, in, s, st, ev);
  }
}

hipError_t launch_route(const LayerDims& d, int m, const Inputs& in, const Scratch& s, hipStream_t st,
                        const KernelEvents& ev) {
  const int groups = (d.E + 63) / 64;  // sort groups; wave w takes w, w+4, ...
  const int gpw = (groups + 3) / 4;
  if (gpw <= 1) return launch_kernel(route_kernel<1>, dim3(m), dim3(kThreads), 0, st, ev, d, m, in.bias, s);
  if (gpw <= 2) return launch_kernel(route_kernel<2>, dim3(m), dim3(kThreads), 0, st, ev, d, m, in.bias, s);
  return launch_kernel(route_kernel<4>, dim3(m), dim3(kThreads), 0, st, ev, d, m, in.bias, s);
}

}  // namespace moe
