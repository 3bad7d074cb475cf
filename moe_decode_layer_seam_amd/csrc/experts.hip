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

__device__ __forceinline__ Frag load_frag_stream(const uint8_t* row, int kw, int g) {
  Frag f;
  f.lo = ld16_stream(row + kw + 16 * g);
  f.hi = ld16_stream(row + kw + 64 + 16 * g);
  return f;
}

__device__ __forceinline__ Frag load_frag(const uint8_t* row, int kw, int g) {
  Frag f;
  f.lo = ld16(row + kw + 16 * g);
  f.hi = ld16(row + kw + 64 + 16 * g);
  return f;
}

// ---------------------------------------------------------------------------
// w13 + SiLU*up + MXFP8
// ---------------------------------------------------------------------------

// Everything one K step (128 columns) of a w13 item needs, per lane.
struct W13Step {
  Frag b[4];   // weight tiles: gate rows 0-15, 16-31, up rows 0-15, 16-31
  Frag a;      // activation rows (token rows of the slot)
  int sa, sg, su;  // E8M0 codes of the lane's K block: activation, gate, up
};

struct W13Item {
  const uint8_t* wrow[4];
  const uint8_t* srow_g;
  const uint8_t* srow_u;
  const uint8_t* xrow;
  const uint8_t* xsrow;
  bool has_tok;
};

__device__ __forceinline__ void w13_load(W13Step& st, const W13Item& it, int step, int g) {
  const int kw = step * 128;
#pragma unroll
  for (int t = 0; t < 4; ++t) st.b[t] = load_frag_stream(it.wrow[t], kw, g);
  st.sg = it.srow_g[4 * step + g];
  st.su = it.srow_u[4 * step + g];
  if (it.has_tok) {
    st.a = load_frag(it.xrow, kw, g);
    st.sa = it.xsrow[4 * step + g];
  } else {
    st.a.lo = u32x4{0, 0, 0, 0};
    st.a.hi = u32x4{0, 0, 0, 0};
    st.sa = 127;
  }
}

__device__ __forceinline__ void w13_mma(v4f (&acc)[4], const W13Step& st) {
  const v8i a = join(st.a.lo, st.a.hi);
  acc[0] = mfma_e4m3(a, join(st.b[0].lo, st.b[0].hi), acc[0], st.sa, st.sg);
  acc[1] = mfma_e4m3(a, join(st.b[1].lo, st.b[1].hi), acc[1], st.sa, st.sg);
  acc[2] = mfma_e4m3(a, join(st.b[2].lo, st.b[2].hi), acc[2], st.sa, st.su);
  acc[3] = mfma_e4m3(a, join(st.b[3].lo, st.b[3].hi), acc[3], st.sa, st.su);
}

__global__ __launch_bounds__(kThreads) void w13_kernel(LayerDims d, Inputs in, Scratch s) {
  __shared__ float red[4][4][16][16];  // [wave][tile][token row][column]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int H = d.H, HB = H / 32, S = H / 128;
  const int s0 = S * wave / 4, s1 = S * (wave + 1) / 4;  // this wave's K steps
  const int n_items = s.header[2], nS = s.header[1];
  const int chS = d.Is / 32, chR = d.I / 32;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
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
    const int ex = slot.x, row0 = slot.y, c = slot.z;
    const int Kv = ex < 0 ? d.Is : d.I;
    const uint8_t* W = ex < 0 ? in.sgu : in.w13 + (size_t)ex * 2 * d.I * H;
    const uint8_t* WS = ex < 0 ? in.sgu_s : in.w13_s + (size_t)ex * (2 * d.I / 32) * HB;

    W13Item it;
    it.wrow[0] = W + (size_t)(32 * chunk + j) * H;
    it.wrow[1] = W + (size_t)(32 * chunk + 16 + j) * H;
    it.wrow[2] = W + (size_t)(Kv + 32 * chunk + j) * H;
    it.wrow[3] = W + (size_t)(Kv + 32 * chunk + 16 + j) * H;
    it.srow_g = WS + (size_t)chunk * HB;
    it.srow_u = WS + (size_t)(Kv / 32 + chunk) * HB;
    it.has_tok = j < c;
    const int tok = it.has_tok ? s.row_tok[row0 + j] : 0;
    it.xrow = s.x8 + (size_t)tok * H;
    it.xsrow = s.x8s + (size_t)tok * HB;

    v4f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

    // double-buffered K loop: step st+1's loads are in flight while step
    // st's MFMAs run
    W13Step f0, f1;
    if (s0 < s1) w13_load(f0, it, s0, g);
    for (int st = s0; st < s1; st += 2) {
      if (st + 1 < s1) w13_load(f1, it, st + 1, g);
      w13_mma(acc, f0);
      if (st + 2 < s1) w13_load(f0, it, st + 2, g);
      if (st + 1 < s1) w13_mma(acc, f1);
    }

#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][t][4 * g + v][j] = acc[t][v];
    __syncthreads();
    {
      // thread -> token row i, intermediate columns 2jj, 2jj+1 of the chunk
      const int i = tid >> 4, jj = tid & 15;
      float av[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col = 2 * jj + q, tg = col >> 4, cc = col & 15;
        float hg = red[0][tg][i][cc] + red[1][tg][i][cc] + red[2][tg][i][cc] + red[3][tg][i][cc];
        float hu = red[0][tg + 2][i][cc] + red[1][tg + 2][i][cc] + red[2][tg + 2][i][cc] + red[3][tg + 2][i][cc];
        av[q] = hg / (1.0f + __expf(-hg)) * hu;
      }
      const float amax = group_max(fmaxf(fabsf(av[0]), fabsf(av[1])), 16);
      const int code = e8m0_code(amax);
      const float mul = mx_mul(code);
      if (i < c) {
        const size_t row = (size_t)(row0 + i);
        *reinterpret_cast<uint16_t*>(s.a8 + row * d.Imax + 32 * chunk + 2 * jj) =
            (uint16_t)fp8x2(av[0] * mul, av[1] * mul);
        if (jj == 0) s.a8s[row * (d.Imax / 32) + chunk] = (uint8_t)code;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// w2 + weighted combine
// ---------------------------------------------------------------------------

template <int SPW>
struct W2Slot {
  Frag b[SPW];
  Frag a[SPW];
  int sa[SPW], sb[SPW];
};

template <int NW, int SPW>
__global__ __launch_bounds__(NW * 64) void w2_kernel(LayerDims d, int m, Inputs in, Scratch s) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int H = d.H, n0 = 16 * blockIdx.x;
  const int nvs = s.header[0];
  const int R = m * d.K + m;

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
  float* my = accl + wave * m * 16;

  for (int v = 0; v < nvs; ++v) {
    const int4 slot = s_vs[v];
    const int ex = slot.x, row0 = slot.y, c = slot.z;
    const int Kv = ex < 0 ? d.Is : d.I;
    const int S = Kv / 128, st0 = S * wave / NW, ns = S * (wave + 1) / NW - st0;
    const uint8_t* wr = (ex < 0 ? in.sw2 : in.w2 + (size_t)ex * H * d.I) + (size_t)(n0 + j) * Kv;
    const uint8_t* sr = (ex < 0 ? in.sw2_s : in.w2_s + (size_t)ex * (H / 32) * (d.I / 32)) +
                        (size_t)(n0 / 32) * (Kv / 32);
    const bool has = j < c;
    const uint8_t* ar = s.a8 + (size_t)(row0 + (has ? j : 0)) * d.Imax;
    const uint8_t* asr = s.a8s + (size_t)(row0 + (has ? j : 0)) * (d.Imax / 32);

    W2Slot<SPW> f;
#pragma unroll
    for (int q = 0; q < SPW; ++q) {
      if (q < ns) {
        const int st = st0 + q, kw = st * 128;
        f.b[q] = load_frag_stream(wr, kw, g);
        f.sb[q] = sr[4 * st + g];
        if (has) {
          f.a[q] = load_frag(ar, kw, g);
          f.sa[q] = asr[4 * st + g];
        } else {
          f.a[q].lo = u32x4{0, 0, 0, 0};
          f.a[q].hi = u32x4{0, 0, 0, 0};
          f.sa[q] = 127;
        }
      }
    }
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < SPW; ++q)
      if (q < ns) acc = mfma_e4m3(join(f.a[q].lo, f.a[q].hi), join(f.b[q].lo, f.b[q].hi), acc, f.sa[q], f.sb[q]);
    if (ns == 0) continue;
    // lane (g, j) holds rows 4g..4g+3 of output column n0 + j
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * g + q;
      if (i < c) {
        const int t = s_tok[row0 + i];
        my[t * 16 + j] += s_w[row0 + i] * acc[q];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < m * 16; idx += NW * 64) {
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += accl[w * m * 16 + idx];
    const int t = idx >> 4, jj = idx & 15;
    in.out[(size_t)t * H + n0 + jj] = (uint16_t)f32_to_bf16(sum);
  }
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

int w13_blocks_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, w13_kernel, kThreads, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

hipError_t launch_w2(const LayerDims& d, int m, const Inputs& in, const Scratch& s, int max_vs, hipStream_t st) {
  constexpr int NW = 4;
  const int steps = (d.Imax / 128 + NW - 1) / NW;  // K steps per wave per slot
  if (steps <= 1) return launch_w2_t<NW, 1>(d, m, in, s, max_vs, st);
  if (steps <= 2) return launch_w2_t<NW, 2>(d, m, in, s, max_vs, st);
  if (steps <= 4) return launch_w2_t<NW, 4>(d, m, in, s, max_vs, st);
  if (steps <= 8) return launch_w2_t<NW, 8>(d, m, in, s, max_vs, st);
  return launch_w2_t<NW, 16>(d, m, in, s, max_vs, st);
}

}  // namespace moe
