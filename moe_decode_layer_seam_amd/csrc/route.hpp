// route.hpp -- the router as block-level device code: per token, sigmoid +
// bias -> top-k -> routing weights, and the token -> expert plan built by the
// last block to finish.  Used by the route launch (seam.hip) and, for steps
// of a few tokens, by the first blocks of the w13 launch (experts.hip).
//
// Pages: "vllm.models.deepseek_v41.amd.mono.runner" MonoLayerWeights (gate_w,
// bias: the e_score_correction_bias), build_mono_ffn (expert groups of 64 for
// the routing sort networks); "vllm.models.deepseek_v41.amd.mono.attention.
// device" atomic_add_dev (relaxed device-scope counters).
#pragma once

#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

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

// The rows of a plan of P <= 64 pairs and at most 16 tokens, by one wave:
// lane p brings pair p's expert (token t's pairs are t k .. t k + k - 1),
// and a bitonic sort of the unique keys expert * 1024 + token * 64 + pair
// leaves row r's pair in lane r.  Every expert has one virtual slot (its rows
// are at most the 16 tokens); `ri` numbers the routed slots from 0.  The same
// rows as build_plan's general path.
struct SmallRows {
  int e, t, p;    // row r = lane: its expert, token and pair
  int cnt, ri;    // where a slot starts: its rows and routed slot index
  int nR;         // routed slots
  bool valid, first;
};

__device__ __forceinline__ SmallRows small_rows(int ex, int P, int K, int lane) {
  int key = 0x7FFFFFFF;
  if (lane < P) key = (ex << 10) | ((lane / K) << 6) | lane;
  // sorted ascending over the smallest power-of-two number of lanes that
  // holds the pairs; every stage unrolled, so each exchange is a fixed DPP
  // or permlane pattern, and a level wider than needed is skipped as a whole
  const int width = P <= 8 ? 8 : (P <= 16 ? 16 : (P <= 32 ? 32 : 64));
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
  SmallRows q;
  const int r = lane;
  q.valid = r < P;
  q.e = key >> 10;
  q.t = (key >> 6) & 15;
  q.p = key & 63;
  const int eprev = __shfl_up(q.e, 1, 64);
  q.first = q.valid && (r == 0 || eprev != q.e);
  const uint64_t fm = __ballot(q.first);
  const uint64_t above = r == 63 ? 0ull : fm & ~((2ull << r) - 1ull);
  q.cnt = (above ? __ffsll((unsigned long long)above) - 1 : P) - r;
  q.nR = __popcll(fm);
  q.ri = __popcll(fm & ((1ull << r) - 1ull));
  return q;
}

// The plan of a step of at most 64 pairs and 16 tokens, by wave 0 alone,
// from the picks in L.ids and L.w (small_rows; slot 0 is the shared
// expert's).
__device__ void plan_small(const LayerDims& d, int m, const Scratch& s, RouteLds& L, int lane) {
  const int K = d.K, P = m * K, nS = 1;
  const SmallRows q = small_rows(lane < P ? L.ids[lane] : 0, P, K, lane);
  const int r = lane;
  if (q.valid) {
    s.row_tok[r] = q.t;
    s.row_w[r] = L.w[q.p];
    s.pair_row[q.p] = r;
    s.row_out[r] = q.p;
  }
  if (q.first) s.vslots[nS + q.ri] = make_int4(q.e, r, q.cnt, 0);
  if (lane < m) {
    s.row_tok[P + lane] = lane;
    s.row_w[P + lane] = 1.0f;
    s.row_out[P + lane] = P + lane;
  }
  if (lane == 0) {
    s.vslots[0] = make_int4(-1, P, m, 0);
    s.header[0] = nS + q.nR;
    s.header[1] = nS;
    s.header[2] = q.nR;
    s.header[3] = m;
    __hip_atomic_store(s.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Tokens per expert of a plan of P <= 64 picks in L.ids, by one wave: a
// table in LDS (L.base) zeroed, counted into and copied out.  One wave's LDS
// operations run in order, so no barrier is needed.
__device__ void plan_counts(const LayerDims& d, int P, const Scratch& s, RouteLds& L, int lane) {
  for (int x = lane; x < d.E; x += 64) L.base[x] = 0;
  if (lane < P) atomicAdd(&L.base[L.ids[lane]], 1);
  for (int x = lane; x < d.E; x += 64) s.counts[x] = L.base[x];
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
  {
    // the other blocks' picks: every load issued before the first is used
    // (one round trip instead of one per kThreads picks)
    constexpr int NL = (kMaxTokens * kMaxTopk + kThreads - 1) / kThreads;
    int idr[NL];
    float wr[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int p = tid + k * kThreads;
      if (p < P && p / K != own) {
        idr[k] = __hip_atomic_load(&s.ids[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wr[k] = __hip_atomic_load(&s.wts[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int p = tid + k * kThreads;
      if (p < P && p / K != own) {
        L.ids[p] = idr[k];
        L.w[p] = wr[k];
      }
    }
  }
  if (P <= 64 && m <= kTokTile) {
    __syncthreads();
    if (threadIdx.x < 64) plan_small(d, m, s, L, threadIdx.x);
    else if (threadIdx.x < 128) plan_counts(d, P, s, L, threadIdx.x - 64);
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

// Exclusive prefix sum of arr[0, n) (n <= 2 * NW * 64) in place by the NW
// waves of a block; returns the total.  tmp: NW ints.
template <int NW>
__device__ int block_scan_w(int* arr, int n, int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int v[2], sum = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = tid * 2 + q;
    v[q] = i < n ? arr[i] : 0;
    sum += v[q];
  }
  int inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    base += w < wave ? tmp[w] : 0;
    total += tmp[w];
  }
  int run = base + inc - sum;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = tid * 2 + q;
    if (i < n) arr[i] = run;
    run += v[q];
  }
  __syncthreads();
  return total;
}

// LDS words plan_block needs beyond the slots and the row map.
inline size_t plan_block_words(int E) { return 4 * (size_t)E + 16; }

// The plan of a step of m tokens from the picks the route launch stored
// (s.ids, s.wts), built by every thread of a block of NW waves with
// build_plan's rows and slots: the slots into s_vs, the token of each row
// into s_tok (both LDS).  With mem, also the plan's arrays in the scratch
// (for the later launches and the taps).  pl: plan_block_words(E) LDS words.
// Returns the number of virtual slots; the LDS is complete on return.
template <int NW>
__device__ int plan_block(const LayerDims& d, int m, const Scratch& s, int4* s_vs, int* s_tok, uint32_t* pl,
                          bool mem) {
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x;
  const int E = d.E, K = d.K, P = m * K;
  uint32_t* mlo = pl;  // tokens 0-31 / 32-47 of each expert
  uint32_t* mhi = pl + E;
  int* base = reinterpret_cast<int*>(pl + 2 * E);
  int* vsb = reinterpret_cast<int*>(pl + 3 * E);
  int* tmp = reinterpret_cast<int*>(pl + 4 * E);
  for (int e = tid; e < E; e += NT) mlo[e] = mhi[e] = 0u;
  __syncthreads();
  for (int p = tid; p < P; p += NT) {
    const int t = p / K, e = s.ids[p];
    if (t < 32) atomicOr(&mlo[e], 1u << t);
    else atomicOr(&mhi[e], 1u << (t - 32));
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    const int c = __popc(mlo[e]) + __popc(mhi[e]);
    base[e] = c;
    vsb[e] = (c + kTokTile - 1) / kTokTile;
    if (mem) s.counts[e] = c;
  }
  __syncthreads();
  block_scan_w<NW>(base, E, tmp);
  const int nR = block_scan_w<NW>(vsb, E, tmp + NW);
  const int nS = (m + kTokTile - 1) / kTokTile;
  for (int p = tid; p < P; p += NT) {
    const int t = p / K, e = s.ids[p];
    const int rank = t < 32 ? __popc(mlo[e] & ((1u << t) - 1u))
                            : __popc(mlo[e]) + __popc(mhi[e] & ((1u << (t - 32)) - 1u));
    const int r = base[e] + rank;
    s_tok[r] = t;
    if (mem) {
      s.row_tok[r] = t;
      s.row_w[r] = s.wts[p];
      s.pair_row[p] = r;
      s.row_out[r] = p;
    }
  }
  for (int e = tid; e < E; e += NT) {
    const int c = __popc(mlo[e]) + __popc(mhi[e]);
    for (int v = 0; v * kTokTile < c; ++v) {
      const int rows = c - v * kTokTile;
      const int4 sl = make_int4(e, base[e] + v * kTokTile, rows < kTokTile ? rows : kTokTile, 0);
      s_vs[nS + vsb[e] + v] = sl;
      if (mem) s.vslots[nS + vsb[e] + v] = sl;
    }
  }
  for (int t = tid; t < m; t += NT) {
    s_tok[P + t] = t;
    if (mem) {
      s.row_tok[P + t] = t;
      s.row_w[P + t] = 1.0f;
      s.row_out[P + t] = P + t;
    }
  }
  for (int v = tid; v < nS; v += NT) {
    const int rows = m - v * kTokTile;
    const int4 sl = make_int4(-1, P + v * kTokTile, rows < kTokTile ? rows : kTokTile, 0);
    s_vs[v] = sl;
    if (mem) s.vslots[v] = sl;
  }
  if (mem && tid == 0) {
    s.header[0] = nS + nR;
    s.header[1] = nS;
    s.header[2] = nR;
    s.header[3] = m;
  }
  __syncthreads();
  return nS + nR;
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

// Block code of the router for token t, run by the first kThreads threads
// of a block of at least kThreads (the others only take part in its
// barriers); nblocks route blocks run in the launch (one per token).
// Returns true in the block that built the plan.  With pbox, each pick is
// also stored there as soon as it is known (kPickBox).  The logits come from
// s.logits, or with lbox from
// the logit box as the blocks of the launch store them (then also copied to
// s.logits).  Wave w sorts the selection
// keys of expert groups w, w + 4, ... (GPW groups of 64) and merges them;
// wave 0 merges the four waves' lists, and its lanes [0, k) hold the picks
// in selection order.
// A logit of the logit box that does not arrive within s.wait_ticks (100 ms
// unless set lower) flags the run (status 2) and is taken as 0.

// The logit at w of the logit box, once it is in.
__device__ __forceinline__ double take_logit(const uint64_t* w, const Scratch& s, uint64_t t0) {
  uint64_t v;
  while ((v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0ull) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > s.wait_ticks) {
      flag_status(s.status, kStatusRouteWait);
      return 0.0;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return __longlong_as_double((long long)(v ^ kLogitTag));
}

// One token's picks by one wave, for at most 64 experts (one sort group):
// the logits read device-coherently from s.logits (other blocks stored them
// through), then route_block's selection keys, network and weights, so the
// ids and weights are route_block's bits.  The picks are stored
// device-coherent for the w13 launch's plan.
__device__ void route_wave(const LayerDims& d, int t, const float* __restrict__ bias, const Scratch& s, int lane) {
  const int E = d.E, K = d.K;
  uint64_t k[1] = {0ull};  // below every real expert's key
  double sg = 0.0;
  if (lane < E) {
    const uint64_t bits = __hip_atomic_load(reinterpret_cast<const uint64_t*>(s.logits) + (size_t)t * E + lane,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const double lg = __longlong_as_double((long long)bits);
    sg = 1.0 / (1.0 + exp(-lg));
    const double bb = sg + (double)bias[lane];
    k[0] = select_key((bb == bb) ? bb : -INFINITY, lane);  // a NaN score ranks last
  }
  sort64<1>(k, lane);
  const int e = 1023 - (int)(k[0] & 0x3FF);
  const double sge = __shfl(sg, e & 63, 64);
  const double sgk = lane < K ? sge : 0.0;
  const double ssum = wave_sum(sgk);
  if (lane < K) {
    const float w = (float)((double)d.routed_scale * sgk / ssum);
    __hip_atomic_store(&s.ids[t * K + lane], e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&s.wts[t * K + lane], w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int GPW>
__device__ bool route_block(const LayerDims& d, int m, int t, int nblocks, const float* __restrict__ bias,
                            const Scratch& s, RouteLds& L, uint32_t* pbox = nullptr,
                            const uint64_t* lbox = nullptr, bool plan = true) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = d.E, K = d.K;
  const int groups = (E + 63) / 64;
  stamp(s.tl_route, kTlPoints, 0);

  uint64_t k[GPW];
  float bx[GPW];  // the biases, loaded before the logits are waited for
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    const int ex = 64 * (wave + 4 * i) + lane;
    bx[i] = (wave < 4 && ex < E) ? bias[ex] : 0.0f;
  }
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    const int ex = 64 * (wave + 4 * i) + lane;
    k[i] = 0;  // below every real expert's key
    if (wave < 4 && ex < E) {
      double lg;
      if (lbox) {
        lg = take_logit(lbox + (size_t)t * E + ex, s, t0);
        s.logits[(size_t)t * E + ex] = lg;
      } else {
        lg = s.logits[(size_t)t * E + ex];
      }
      const double sg = 1.0 / (1.0 + exp(-lg));
      const double bb = sg + (double)bx[i];
      L.sig[ex] = sg;
      k[i] = select_key((bb == bb) ? bb : -INFINITY, ex);  // a NaN score ranks last
    }
  }
  stamp(s.tl_route, kTlPoints, 5);
  if (wave < groups && wave < 4) {
    sort64<GPW>(k, lane);
#pragma unroll
    for (int width = GPW / 2; width >= 1; width >>= 1) {
#pragma unroll
      for (int i = 0; i < width; ++i) merge64(k[i], k[i + width], lane);
    }
  }
  if (wave < 4) L.cand[wave][lane] = k[0];
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
    // the w13 launch's blocks wait for the picks alone: stored first
    if (pbox && lane < K) store_coherent(pbox + t * K + lane, kBoxTag | (uint32_t)e);
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
  // without plan, the launch after this one builds it from the stored picks
  if (!plan) return false;
  if (nblocks == 1 && K <= 64) {
    // one token: wave 0 holds every pick and builds the plan from them
    // straight away (its own LDS writes, in order; no barrier)
    if (wave == 0) {
      plan_small(d, 1, s, L, lane);
      plan_counts(d, K, s, L, lane);
    }
    stamp(s.tl_route, kTlPoints, 4);
    return true;
  }

  if (nblocks > 1) {
    // Arrival: wait until this block's coherent stores completed, count the
    // block, and let the last one through to the plan.  Nothing spins.  (A
    // workgroup-scope fence would not wait for the stores: only the explicit
    // wait orders them before the count.)
    wait_memory();
    __syncthreads();
    if (tid == 0)
      L.last = (__hip_atomic_fetch_add(s.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)(nblocks - 1));
    __syncthreads();
    if (!L.last) return false;
  } else {
    __syncthreads();
  }
  stamp(s.tl_route, kTlPoints, 3);
  build_plan(d, m, t, s, L);
  stamp(s.tl_route, kTlPoints, 4);
  return true;
}


}  // namespace
}  // namespace moe
