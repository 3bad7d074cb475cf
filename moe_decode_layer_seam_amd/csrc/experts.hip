// experts.hip -- the expert GEMMs on the gfx950 scaled MFMA (E4M3 x E4M3,
// 32 x 32 E8M0 weight blocks, 16x16x128 per instruction).
//
//   w13: for every (virtual slot, 32-column chunk of the intermediate) item,
//        h = x8 . W13^T over the chunk's 32 gate and 32 up rows, then
//        a = SiLU(gate) * up and its MXFP8 (a8, a8s) per 32 columns.
//   w2:  for every 16-row tile of the output, y = a8 . W2^T of every virtual
//        slot, weighted by its rows' routing weights and summed into the
//        token rows in a fixed order, then rounded to bf16 once.
//
// Pages: "vllm.models.deepseek_v41.amd.mono.runner" MonoLayerWeights (w13
// [E, 2I, H] gate/up, w2 [E, H, I], sgu, sw2, their 32 x 32 E8M0 scales);
// "vllm.models.deepseek_v41.amd.mono.attention.device" mfma_scaled (lane
// layout of the scaled MFMA), mx_code / fp8_pack4 (the requantisation);
// "vllm.models.deepseek_v41.amd.mono.layer" run_ffn (the MoE's output).
//
// Weights are streamed once, straight from HBM into MFMA operand registers:
// each load instruction reads 64 contiguous bytes of 16 rows, the layout the
// MFMA wants, so no LDS staging is needed for a tile that is used once.
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// One 128-byte K window of one lane's row: the two 16-byte pieces the
// scaled MFMA wants in its first and second register halves.
struct Frag {
  u32x4 lo, hi;
};

// ---------------------------------------------------------------------------
// w13 + SiLU*up + MXFP8
// ---------------------------------------------------------------------------

// Everything one K step (128 columns) of a w13 item needs, per lane.
struct W13Step {
  Frag b[4];       // weight tiles: gate rows 0-15, 16-31, up rows 0-15, 16-31
  Frag a;          // activation rows (token rows of the slot; zero past them)
  int sa, sg, su;  // E8M0 codes of the lane's K block: activation, gate, up
};

// One item's buffers: the expert's w13 and its codes, the MXFP8 rows.  Tile
// t's rows start at soff[t] (bytes) inside the expert; lane (g, j) reads row
// j of each tile at column kw + 16 g (+ 64).
struct W13Item {
  rsrc_t w, ws, x, xs;
  uint32_t soff[4], sg_off, su_off;
  uint32_t wlane, row8, slane, xlane, xslane;
  int row0, c, chunk;
};

// Loads of K step `step` (kNoRow offsets past the segment: zeros, no traffic).
// Weights come as whole 128-byte lines (b[t].lo = rows 0-7, b[t].hi = rows
// 8-15, rearranged by lines_to_mfma before use).
__device__ __forceinline__ void w13_load(W13Step& st, const W13Item& it, int step, bool ok) {
  const uint32_t kw = step * 128;
  const uint32_t wo = ok ? it.wlane + kw : kNoRow;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    st.b[t].lo = bload16_nt(it.w, wo, it.soff[t]);
    st.b[t].hi = bload16_nt(it.w, wo, it.soff[t] + it.row8);
  }
  const uint32_t so = ok ? it.slane + 4 * step : kNoRow;
  st.sg = bload8(it.ws, so, it.sg_off);
  st.su = bload8(it.ws, so, it.su_off);
  const uint32_t xo = ok ? it.xlane + kw : kNoRow;
  st.a.lo = bload16(it.x, xo, 0);
  st.a.hi = bload16(it.x, xo + 64, 0);
  st.sa = bload8(it.xs, ok ? it.xslane + 4 * step : kNoRow, 0);
}

__device__ __forceinline__ void w13_mma(v4f (&acc)[4], const W13Step& st) {
  const v8i a = join(st.a.lo, st.a.hi);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    u32x4 lo, hi;
    lines_to_mfma(st.b[t].lo, st.b[t].hi, lo, hi);
    acc[t] = mfma_e4m3(a, join(lo, hi), acc[t], st.sa, t < 2 ? st.sg : st.su);
  }
}

// Item = (virtual slot, 32-column chunk of the intermediate): the chunk's 32
// gate rows and 32 up rows of the slot's expert, for the slot's token rows.
__device__ __forceinline__ W13Item w13_item(int item, const LayerDims& d, const Inputs& in, const Scratch& s,
                                            int m, int g, int j) {
  const int H = d.H, HB = H / 32;
  const int nS = s.header[1], chS = d.Is / 32, chR = d.I / 32;
  int vs, chunk;
  if (item < nS * chS) {
    vs = item / chS;
    chunk = item % chS;
  } else {
    const int r = item - nS * chS;
    vs = nS + r / chR;
    chunk = r % chR;
  }
  const int4 slot = s.vslots[vs];
  const int ex = slot.x;
  const int Kv = ex < 0 ? d.Is : d.I;
  const uint8_t* W = ex < 0 ? in.sgu : in.w13 + (size_t)ex * 2 * d.I * H;
  const uint8_t* WS = ex < 0 ? in.sgu_s : in.w13_s + (size_t)ex * (2 * d.I / 32) * HB;
  W13Item it;
  it.row0 = slot.y;
  it.c = slot.z;
  it.chunk = chunk;
  it.w = make_rsrc(W, (uint32_t)(2 * Kv) * H);
  it.ws = make_rsrc(WS, (uint32_t)(2 * Kv / 32) * HB);
  it.x = make_rsrc(s.x8, (uint32_t)m * H);
  it.xs = make_rsrc(s.x8s, (uint32_t)m * HB);
  it.soff[0] = (uint32_t)(32 * chunk) * H;
  it.soff[1] = (uint32_t)(32 * chunk + 16) * H;
  it.soff[2] = (uint32_t)(Kv + 32 * chunk) * H;
  it.soff[3] = (uint32_t)(Kv + 32 * chunk + 16) * H;
  it.sg_off = (uint32_t)chunk * HB;
  it.su_off = (uint32_t)(Kv / 32 + chunk) * HB;
  it.wlane = (uint32_t)(j & 7) * H + (j < 8 ? 16 * g : 64 + 16 * g);
  it.row8 = (uint32_t)8 * H;
  it.slane = (uint32_t)g;  // the lane group's 32-column K block
  const int tok = j < it.c ? s.row_tok[it.row0 + j] : -1;
  it.xlane = tok >= 0 ? (uint32_t)tok * H + 16 * g : kNoRow;
  it.xslane = tok >= 0 ? (uint32_t)tok * HB + g : kNoRow;
  return it;
}

// SiLU(gate) * up of the item's 32 columns and their MXFP8, from the full
// sums: lane (g, j) holds token rows 4g..4g+3 of gate columns j (tile 0) and
// 16 + j (tile 1) and the same up columns (tiles 2, 3); the 16 lanes of a
// lane group hold one token row's 32 columns.
__device__ __forceinline__ void w13_epilogue(const v4f (&acc)[4], const W13Item& it, const LayerDims& d,
                                             const Scratch& s, int g, int j) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float g0 = acc[0][v], g1 = acc[1][v];
    const float a0 = g0 / (1.0f + __expf(-g0)) * acc[2][v];
    const float a1 = g1 / (1.0f + __expf(-g1)) * acc[3][v];
    const float amax = group_max(fmaxf(fabsf(a0), fabsf(a1)), 16);
    const int code = e8m0_code(amax);
    const float mul = mx_mul(code);
    const int i = 4 * g + v;
    if (i < it.c) {
      const uint32_t q = fp8x2(a0 * mul, a1 * mul);
      const size_t row = (size_t)(it.row0 + i);
      uint8_t* dst = s.a8 + row * d.Imax + 32 * it.chunk;
      dst[j] = (uint8_t)(q & 0xFF);
      dst[16 + j] = (uint8_t)(q >> 8);
      if (j == 0) s.a8s[row * (d.Imax / 32) + it.chunk] = (uint8_t)code;
    }
  }
}

// The worker (wave) whose share of the T (item, K step) pairs holds pair p,
// for W workers with shares [floor(T w / W), floor(T (w + 1) / W)).
__device__ __forceinline__ int worker_of(int64_t p, int64_t T, int64_t W) { return (int)(((p + 1) * W - 1) / T); }
__device__ __forceinline__ int64_t share_begin(int w, int64_t T, int64_t W) { return T * w / W; }

// Stream-K over waves: the n_items x S (item, K step) pairs are cut into
// equal contiguous shares, one per wave, so every CU streams the same bytes
// whatever the routing.  A wave owning a whole item finishes it (SiLU*up and
// the MXFP8 of the result); of an item split between waves each wave stores
// its partial sums, which the next launch (w13_finish_kernel) adds up in wave
// order.  Nothing in this kernel waits on another wave.
// Three 256-thread blocks per CU (at most 168 VGPRs a lane).
constexpr int kW13Burst = 2;
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void w13_kernel(LayerDims d, Inputs in, Scratch s) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int S = d.H / 128;
  const int m = s.header[3];
  const int64_t T = (int64_t)s.header[2] * S;
  const int64_t Wl = (int64_t)gridDim.x * 4;
  const int64_t W = T < Wl ? T : Wl;
  const int w = blockIdx.x * 4 + wave;
  stamp(s.tl_w13, kTlPoints, 0);
  if (w >= W) return;  // no barrier in this kernel: waves are independent
  const int64_t begin = share_begin(w, T, W), end = share_begin(w + 1, T, W);
  const int first_item = (int)(begin / S);

  for (int64_t pos = begin; pos < end;) {
    const int item = (int)(pos / S);
    const int sa = (int)(pos % S);
    const int sb = (end - pos) < (int64_t)(S - sa) ? sa + (int)(end - pos) : S;
    const W13Item it = w13_item(item, d, in, s, m, g, j);

    v4f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
    // K loop in bursts of kW13Burst steps: every load of the burst is issued
    // before its first MFMA (steps past the segment read zeros and add
    // nothing), with no condition inside the loop body.
    for (int st = sa; st < sb; st += kW13Burst) {
      W13Step f[kW13Burst];
#pragma unroll
      for (int u = 0; u < kW13Burst; ++u) w13_load(f[u], it, st + u, st + u < sb);
      __builtin_amdgcn_sched_barrier(0);  // the whole burst in flight first
#pragma unroll
      for (int u = 0; u < kW13Burst; ++u) w13_mma(acc, f[u]);
      __builtin_amdgcn_sched_barrier(0);
    }

    if (sa == 0 && sb == S) {
      w13_epilogue(acc, it, d, s, g, j);
    } else {
      // partial sums of the item's live token rows: slot 0 for the wave's
      // first item, 1 for its last
      float* mine = s.part + ((size_t)2 * w + (item == first_item ? 0 : 1)) * (kTokTile * 64);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (4 * g + v < it.c) mine[(4 * g + v) * 64 + 16 * t + j] = acc[t][v];
    }
    if (pos == begin) stamp(s.tl_w13, kTlPoints, 1);
    pos += sb - sa;
  }
  stamp(s.tl_w13, kTlPoints, 2);
  stamp_wave(s.tl_w13, kTlPoints, 3 + wave);
}

// One wave per item split by w13_kernel (w13_waves: that launch's waves):
// the partial sums of its waves added in wave order, then SiLU*up and the
// MXFP8 of the result.
__global__ __launch_bounds__(kThreads) void w13_finish_kernel(LayerDims d, Inputs in, Scratch s, int w13_waves) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int S = d.H / 128;
  const int n_items = s.header[2], m = s.header[3];
  const int64_t T = (int64_t)n_items * S;
  const int64_t W = T < (int64_t)w13_waves ? T : (int64_t)w13_waves;
  const int item = blockIdx.x * 4 + wave;
  stamp(s.tl_w13f, kTlPoints, 0);
  if (item >= n_items) return;
  const int wf = worker_of((int64_t)item * S, T, W), wl = worker_of((int64_t)(item + 1) * S - 1, T, W);
  if (wf == wl) return;  // finished by its one wave
  const W13Item it = w13_item(item, d, in, s, m, g, j);
  v4f tot[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) tot[t] = v4f{0.f, 0.f, 0.f, 0.f};
  // the shares' loads in batches of 4 waves, added in wave order
  for (int w0 = wf; w0 <= wl; w0 += 4) {
    float v[4][4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ww = w0 + q;
      const int fi = (int)(share_begin(ww <= wl ? ww : wl, T, W) / S);
      const float* src = s.part + ((size_t)2 * (ww <= wl ? ww : wl) + (item == fi ? 0 : 1)) * (kTokTile * 64);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[q][t][r] = (ww <= wl && 4 * g + r < it.c) ? src[(4 * g + r) * 64 + 16 * t + j] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (w0 + q <= wl)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) tot[t][r] += v[q][t][r];
  }
  w13_epilogue(tot, it, d, s, g, j);
  stamp(s.tl_w13f, kTlPoints, 1);
}

// ---------------------------------------------------------------------------
// w2 + weighted combine
// ---------------------------------------------------------------------------

template <int SPW>
struct W2Part {
  Frag b[SPW];
  Frag a[SPW];
  int sa[SPW], sb[SPW];
  int ns, c, row0;
};

// Walks this wave's share of every virtual slot in parts of at most SPW K
// steps: (slot v, first step of the part).
struct W2Cursor {
  int v, st, end;
};

template <int NW>
__device__ __forceinline__ void w2_cursor_enter(W2Cursor& k, const int4* s_vs, int nvs, const LayerDims& d,
                                                int wave) {
  // advance to the next slot with work for this wave
  while (k.v < nvs) {
    const int Kv = s_vs[k.v].x < 0 ? d.Is : d.I;
    const int S = Kv / 128;
    k.st = S * wave / NW;
    k.end = S * (wave + 1) / NW;
    if (k.st < k.end) return;
    ++k.v;
  }
}

template <int NW, int SPW>
__device__ __forceinline__ bool w2_load(W2Part<SPW>& f, W2Cursor& k, const int4* s_vs, int nvs,
                                        const LayerDims& d, const Inputs& in, const Scratch& s, int m, int n0,
                                        int wave, int g, int j) {
  if (k.v >= nvs) {
    f.ns = 0;
    return false;
  }
  const int4 slot = s_vs[k.v];
  const int ex = slot.x;
  f.row0 = slot.y;
  f.c = slot.z;
  const int Kv = ex < 0 ? d.Is : d.I;
  const int rem = k.end - k.st;
  f.ns = rem < SPW ? rem : SPW;
  const rsrc_t wr = make_rsrc(ex < 0 ? in.sw2 : in.w2 + (size_t)ex * d.H * d.I, (uint32_t)d.H * Kv);
  const rsrc_t sr = make_rsrc(ex < 0 ? in.sw2_s : in.w2_s + (size_t)ex * (d.H / 32) * (d.I / 32),
                              (uint32_t)(d.H / 32) * (Kv / 32));
  const uint32_t R = (uint32_t)(m * d.K + m);
  const rsrc_t ar = make_rsrc(s.a8, R * d.Imax);
  const rsrc_t asr = make_rsrc(s.a8s, R * (d.Imax / 32));
  const uint32_t wlane = (uint32_t)(n0 + j) * Kv + 16 * g;
  const uint32_t slane = (uint32_t)(n0 / 32) * (Kv / 32) + g;
  const bool has = j < f.c;
  const uint32_t alane = has ? (uint32_t)(f.row0 + j) * d.Imax + 16 * g : kNoRow;
  const uint32_t aslane = has ? (uint32_t)(f.row0 + j) * (d.Imax / 32) + g : kNoRow;
#pragma unroll
  for (int q = 0; q < SPW; ++q) {
    if (q < f.ns) {
      const uint32_t st = k.st + q, kw = st * 128;
      f.b[q].lo = bload16(wr, wlane + kw, 0);
      f.b[q].hi = bload16(wr, wlane + kw + 64, 0);
      f.sb[q] = bload8(sr, slane + 4 * st, 0);
      f.a[q].lo = bload16(ar, alane + kw, 0);
      f.a[q].hi = bload16(ar, alane + kw + 64, 0);
      f.sa[q] = bload8(asr, aslane + 4 * st, 0);
    }
  }
  k.st += f.ns;
  if (k.st >= k.end) {
    ++k.v;
    w2_cursor_enter<NW>(k, s_vs, nvs, d, wave);
  }
  return true;
}

// MFMAs of a loaded part, then its weighted rows added into the wave's
// per-token accumulator (lane (g, j) holds rows 4g..4g+3 of column n0 + j).
template <int SPW>
__device__ __forceinline__ void w2_use(const W2Part<SPW>& f, float* my, const int* s_tok, const float* s_w,
                                       int g, int j) {
  if (f.ns == 0) return;
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < SPW; ++q)
    if (q < f.ns) acc = mfma_e4m3(join(f.a[q].lo, f.a[q].hi), join(f.b[q].lo, f.b[q].hi), acc, f.sa[q], f.sb[q]);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * g + q;
    if (i < f.c) {
      const int t = s_tok[f.row0 + i];
      my[t * 16 + j] += s_w[f.row0 + i] * acc[q];
    }
  }
}

template <int NW, int SPW>
__global__ __launch_bounds__(NW * 64) void w2_kernel(LayerDims d, int m, Inputs in, Scratch s) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int H = d.H, n0 = 16 * blockIdx.x;
  const int nvs = s.header[0];
  const int R = m * d.K + m;
  stamp(s.tl_w2, kTlPoints, 0);

  float* accl = reinterpret_cast<float*>(lds_raw);  // [NW][m][16]
  int4* s_vs = reinterpret_cast<int4*>(accl + NW * m * 16);
  int* s_tok = reinterpret_cast<int*>(s_vs + nvs);
  float* s_w = reinterpret_cast<float*>(s_tok + R);
  for (int i = tid; i < NW * m * 16; i += NW * 64) accl[i] = 0.0f;
  for (int i = tid; i < nvs; i += NW * 64) s_vs[i] = s.vslots[i];
  for (int i = tid; i < R; i += NW * 64) {
    s_tok[i] = s.row_tok[i];
    s_w[i] = s.row_w[i];
  }
  __syncthreads();
  stamp(s.tl_w2, kTlPoints, 1);
  float* my = accl + wave * m * 16;

  // two parts in flight: part p+1's loads are issued before part p's MFMAs
  W2Cursor k{0, 0, 0};
  w2_cursor_enter<NW>(k, s_vs, nvs, d, wave);
  W2Part<SPW> f0, f1;
  bool more = w2_load<NW, SPW>(f0, k, s_vs, nvs, d, in, s, m, n0, wave, g, j);
  while (more) {
    const bool more1 = w2_load<NW, SPW>(f1, k, s_vs, nvs, d, in, s, m, n0, wave, g, j);
    w2_use<SPW>(f0, my, s_tok, s_w, g, j);
    if (!more1) break;
    more = w2_load<NW, SPW>(f0, k, s_vs, nvs, d, in, s, m, n0, wave, g, j);
    w2_use<SPW>(f1, my, s_tok, s_w, g, j);
  }
  __syncthreads();
  stamp(s.tl_w2, kTlPoints, 2);
  for (int idx = tid; idx < m * 16; idx += NW * 64) {
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += accl[w * m * 16 + idx];
    const int t = idx >> 4, jj = idx & 15;
    in.out[(size_t)t * H + n0 + jj] = (uint16_t)f32_to_bf16(sum);
  }
  stamp(s.tl_w2, kTlPoints, 3);
}

template <int NW, int SPW>
hipError_t launch_w2_t(const LayerDims& d, int m, const Inputs& in, const Scratch& s, int max_vs, hipStream_t st) {
  const size_t lds = (size_t)NW * m * 16 * 4 + (size_t)max_vs * 16 + (size_t)(m * d.K + m) * 8;
  hipLaunchKernelGGL((w2_kernel<NW, SPW>), dim3(d.H / 16), dim3(NW * 64), lds, st, d, m, in, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w13(const LayerDims& d, int /*m*/, const Inputs& in, const Scratch& s, int grid, hipStream_t st) {
  hipLaunchKernelGGL(w13_kernel, dim3(grid), dim3(kThreads), 0, st, d, in, s);
  return hipGetLastError();
}

hipError_t launch_w13_finish(const LayerDims& d, int m, const Inputs& in, const Scratch& s, int w13_grid,
                             hipStream_t st) {
  const int max_items = max_vslots(m, d.E, d.K) * (d.Imax / 32);
  hipLaunchKernelGGL(w13_finish_kernel, dim3((max_items + 3) / 4), dim3(kThreads), 0, st, d, in, s, w13_grid * 4);
  return hipGetLastError();
}

int w13_blocks_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, w13_kernel, kThreads, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

hipError_t launch_w2(const LayerDims& d, int m, const Inputs& in, const Scratch& s, int max_vs, hipStream_t st) {
  constexpr int NW = 8;
  const int steps = (d.Imax / 128 + NW - 1) / NW;  // K steps per wave per slot
  // parts of at most four K steps; longer shares are walked part by part
  if (steps <= 1) return launch_w2_t<NW, 1>(d, m, in, s, max_vs, st);
  if (steps <= 2) return launch_w2_t<NW, 2>(d, m, in, s, max_vs, st);
  return launch_w2_t<NW, 4>(d, m, in, s, max_vs, st);
}

}  // namespace moe
