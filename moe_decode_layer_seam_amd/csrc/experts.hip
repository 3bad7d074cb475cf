// experts.hip -- the expert GEMMs on the gfx950 scaled MFMA (E4M3 x E4M3,
// 32 x 32 E8M0 weight blocks, 16x16x128 per instruction) and the two small
// kernels that finish them:
//
//   w13:     h = x8 . W13^T of every virtual slot (an expert's token rows,
//            at most 16 of them, or the shared expert's), fp32
//   act:     a = SiLU(h_gate) * h_up and its MXFP8 (a8, a8s) per 32 columns
//   w2:      y = a8 . W2^T of every virtual slot, fp32
//   combine: out[t] = bf16(sum_j w_tj y[row(t, j)] + y[shared row of t])
//
// Pages: "vllm.models.deepseek_v41.amd.mono.runner" MonoLayerWeights (w13
// [E, 2I, H] gate/up, w2 [E, H, I], sgu, sw2, their 32 x 32 E8M0 scales);
// "vllm.models.deepseek_v41.amd.mono.attention.device" mfma_scaled (lane
// layout of the scaled MFMA), mx_code / fp8_pack4 (the requantisation);
// "vllm.models.deepseek_v41.amd.mono.layer" run_ffn (the MoE's output).
//
// Arithmetic.  Each GEMM output tile is 16 weight rows x a slot's token rows.
// Its K range is cut into fixed segments of kSegSteps K steps; a segment's
// sum starts from zero and runs through its MFMAs in K order, and the tile's
// value is the segments' sums added in segment order.  That order depends
// only on the layer's shape, never on m or on which wave did the work, so a
// token's result is the same bits whatever batch it is in.
//
// Schedule.  The weights are streamed once, straight from HBM into MFMA
// operand registers (whole 128-byte lines, rearranged with DPP), by one block
// per CU.  Work is cut into units: a whole tile when there are many tiles
// (its segment sums are added in registers), one segment of a tile when there
// are few (at small m: then the segment sums are stored and the next kernel
// adds them, in the same order).  Each CU takes an equal share of the units;
// inside a CU, fast waves take more of them.
#include <cmath>

#include "device.hpp"
#include "kernels.hpp"
#include "route.hpp"

namespace moe {
namespace {

// Geometry of one GEMM for one kind of slot (shared or routed expert).
struct Geo {
  int tiles;  // 16-row weight tiles
  int K;      // bytes per weight row (the contraction length)
  int seg;    // K steps per segment
  int nseg;   // K segments
};

template <bool W13>
__device__ __forceinline__ Geo geo(const LayerDims& d, bool shared) {
  const int Kv = shared ? d.Is : d.I;
  Geo g;
  g.tiles = W13 ? 2 * Kv / 16 : d.H / 16;
  g.K = W13 ? d.H : Kv;
  g.seg = W13 ? kSegSteps : w2_seg_steps(d, Kv, !shared && d.rfmt == MOE_DECODE_ROUTED_MXFP4);
  g.nseg = (g.K / 128 + g.seg - 1) / g.seg;
  return g;
}

// The dynamic LDS of the GEMM launches (slots, row map, and in the launch
// that routes the MXFP8 rows), addressed by byte offset.
extern __shared__ __align__(16) unsigned char dyn_lds[];
__device__ __forceinline__ u32x4 lds16(uint32_t o) { return *reinterpret_cast<const u32x4*>(dyn_lds + o); }
__device__ __forceinline__ uint32_t lds32(uint32_t o) { return *reinterpret_cast<const uint32_t*>(dyn_lds + o); }

// One K step of a lane for TT weight tiles: each tile's lines (x: rows 0-7,
// y: rows 8-15), the activation fragment they share, and the E8M0 codes of
// the lane group's K block (one weight code per pair of tiles).
template <int TT>
struct Step {
  u32x4 x[TT], y[TT], alo, ahi;
  int sa, sb[TT / 2];
};

// The operands of one unit, per lane (g, j): TT consecutive 16-row weight
// tiles starting at weight row col0, and the slot's activation row j.
struct UnitOps {
  rsrc_t w, ws, a, as;
  uint32_t wsoff, wlane, row8, tstride, ssoff, sstride, slane, alane, aslane;
  int row0, c, col0, nsteps, seg;
  int fp4;  // weights as E2M1 pairs with per-row 32-column codes, blocked
};

// ALDS (w13 of the launch that routes): the activation rows are the MXFP8
// in the block's LDS, values at byte x8o, codes at xso; alane and aslane are
// then LDS offsets.
template <bool W13, int TT, bool ALDS = false>
__device__ __forceinline__ UnitOps unit_ops(const int4& slot, int tgroup, const LayerDims& d, const Inputs& in,
                                            const Scratch& s, const int* s_tok, int m, int R, int g, int j,
                                            uint32_t x8o = 0, uint32_t xso = 0) {
  // A unit is one wave's: its slot and tile group are the same in every
  // lane.  Read as such, the weight and code descriptors built from them
  // stay in scalar registers; where the compiler could not prove it (slots
  // read back from the LDS), every buffer load went into a loop over the
  // lanes' distinct descriptors.
  const int ex = __builtin_amdgcn_readfirstlane(slot.x);
  tgroup = __builtin_amdgcn_readfirstlane(tgroup);
  const bool shared = ex < 0;
  const Geo G = geo<W13>(d, shared);
  const int N = 16 * G.tiles;
  const uint8_t* W;
  const uint8_t* WS;
  UnitOps u;
  u.fp4 = !shared && d.rfmt == MOE_DECODE_ROUTED_MXFP4;
  // bytes per weight row and codes per weight row block (E4M3: one per 32
  // rows; E2M1: one per row)
  const uint32_t rowb = u.fp4 ? G.K / 2 : G.K;
  if (W13) {
    W = shared ? in.sgu : in.w13 + (size_t)ex * 2 * d.I * (d.H / (u.fp4 ? 2 : 1));
    WS = shared ? in.sgu_s : in.w13_s + (size_t)ex * (u.fp4 ? (size_t)(2 * d.I / 16) * G.nseg * 256
                                                          : (size_t)(2 * d.I / 32) * (d.H / 32));
  } else {
    W = shared ? in.sw2 : in.w2 + (size_t)ex * d.H * (d.I / (u.fp4 ? 2 : 1));
    WS = shared ? in.sw2_s : in.w2_s + (size_t)ex * (u.fp4 ? (size_t)(d.H / 16) * G.nseg * 256
                                                         : (size_t)(d.H / 32) * (d.I / 32));
  }
  u.row0 = __builtin_amdgcn_readfirstlane(slot.y);
  u.c = __builtin_amdgcn_readfirstlane(slot.z);
  u.col0 = 16 * TT * tgroup;
  u.nsteps = G.K / 128;
  u.seg = G.seg;
  u.w = make_rsrc(W, (uint32_t)N * rowb);
  u.ws = make_rsrc(WS, u.fp4 ? (uint32_t)G.tiles * G.nseg * 256 : (uint32_t)(N / 32) * (G.K / 32));
  u.wsoff = (uint32_t)u.col0 * rowb;
  u.tstride = (uint32_t)16 * rowb;
  u.wlane = (uint32_t)(j & 7) * rowb + (j < 8 ? 16 * g : 64 + 16 * g);
  u.row8 = (uint32_t)8 * rowb;
  if (u.fp4) {
    // codes blocked [tile][segment][16 rows][16 blocks]: 256 bytes per tile
    // and segment
    u.ssoff = (uint32_t)(u.col0 / 16) * G.nseg * 256;  // the tile group's first tile
    u.sstride = (uint32_t)G.nseg * 256;                // per tile
    u.slane = (uint32_t)j * 16 + 4 * g;                // the lane's row, blocks 4 g .. 4 g + 3
  } else {
    u.ssoff = (uint32_t)(u.col0 / 32) * (G.K / 32);  // the first tile pair's 32-row code block
    u.sstride = (uint32_t)(G.K / 32);
    u.slane = (uint32_t)g;  // the lane group's 32-column K block
  }
  if (W13) {
    const int tok = j < u.c ? s_tok[u.row0 + j] : -1;
    u.a = make_rsrc(s.x8, (uint32_t)m * d.H);
    u.as = make_rsrc(s.x8s, (uint32_t)m * (d.H / 32));
    u.alane = tok >= 0 ? (ALDS ? x8o : 0u) + (uint32_t)tok * d.H + 16 * g : kNoRow;
    u.aslane = tok >= 0 ? (ALDS ? xso : 0u) + (uint32_t)tok * (d.H / 32) + g : kNoRow;
  } else {
    const uint32_t r = (uint32_t)(u.row0 + j);
    u.a = make_rsrc(s.a8, (uint32_t)R * d.Imax);
    u.as = make_rsrc(s.a8s, (uint32_t)R * (d.Imax / 32));
    u.alane = j < u.c ? r * d.Imax + 16 * g : kNoRow;
    u.aslane = j < u.c ? r * (d.Imax / 32) + g : kNoRow;
  }
  return u;
}

// Loads of K step `st` (past the contraction: zeros, no traffic); AUX: the
// cache policy of the activation loads.
template <int TT, int AUX, bool ALDS>
__device__ __forceinline__ void load_step(Step<TT>& f, const UnitOps& u, int st) {
  const bool ok = st < u.nsteps;
  const uint32_t kw = (uint32_t)st * 128;
  const uint32_t wo = ok ? u.wlane + kw : kNoRow;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    f.x[t] = bload16_nt(u.w, wo, u.wsoff + t * u.tstride);
    f.y[t] = bload16_nt(u.w, wo, u.wsoff + t * u.tstride + u.row8);
  }
  const uint32_t so = ok ? u.slane + 4 * st : kNoRow;
#pragma unroll
  for (int p = 0; p < TT / 2; ++p) f.sb[p] = bload8(u.ws, so, u.ssoff + p * u.sstride);
  if constexpr (ALDS) {
    const bool ar = ok && u.alane != kNoRow;
    f.alo = ar ? lds16(u.alane + kw) : u32x4{0u, 0u, 0u, 0u};
    f.ahi = ar ? lds16(u.alane + kw + 64) : u32x4{0u, 0u, 0u, 0u};
    f.sa = ar ? (int)dyn_lds[u.aslane + 4 * st] : 0;
  } else {
    const uint32_t ao = ok ? u.alane + kw : kNoRow;
    f.alo = bload16a<AUX>(u.a, ao, 0);
    f.ahi = bload16a<AUX>(u.a, ao + 64, 0);
    f.sa = bload8a<AUX>(u.as, ok ? u.aslane + 4 * st : kNoRow, 0);
  }
}

// One segment's sums for the TT tiles (SEG K steps), in bursts of BS K
// steps: a burst's loads are all issued before its first MFMA.  Each tile's
// MFMAs run in K order whatever BS is.
template <int TT, int BS, int AUX, bool ALDS, int SEG>
__device__ __forceinline__ void segment_sum(v4f (&acc)[TT], const UnitOps& u, int seg) {
  static_assert(SEG % BS == 0, "bursts tile the segment");
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b0 = 0; b0 < SEG; b0 += BS) {
    Step<TT> f[BS];
#pragma unroll
    for (int q = 0; q < BS; ++q) load_step<TT, AUX, ALDS>(f[q], u, seg * SEG + b0 + q);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < BS; ++q) {
      const v8i a = join(f[q].alo, f[q].ahi);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        u32x4 lo, hi;
        lines_to_mfma(f[q].x[t], f[q].y[t], lo, hi);
        acc[t] = mfma_e4m3(a, join(lo, hi), acc[t], f[q].sa, f[q].sb[t / 2]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// E2M1 weights: one 128-byte line of a row holds two K steps (64 bytes
// each).  Lane (g, j) of load X reads row j & 7 of the tile at step st + (j
// >= 8) bytes [16 g, +16), load Y the same for rows 8..15; the DPP row shifts
// of lines_to_mfma give every lane its row's step st operand in `lo` and
// step st + 1 in `hi`.
template <int TT>
struct Pair4 {
  u32x4 x[TT], y[TT], alo[2], ahi[2];
};

// The segment's E8M0 codes, one word per lane and tile: byte s = the code of
// step s of the segment for the lane's row and its lane group's K block.
// Each lane loads the four codes of step g (blocks 4 g .. 4 g + 3 of its
// row's 16 in the segment); a byte transpose across the lane groups turns
// that into the four steps of its own block.
template <int TT>
struct Codes4 {
  uint32_t b[TT], a;
};

template <int TT, int AUX, bool ALDS>
__device__ __forceinline__ void load_codes4(Codes4<TT>& c, const UnitOps& u, int seg, int g) {
  const int st = seg * kSegSteps + g;  // the step whose codes this lane fetches
  const bool ok = st < u.nsteps;
  // the lane's row, blocks 4 g .. 4 g + 3 of the segment (step seg * 4 + g):
  // the whole wave reads the segment's 256-byte code block of each tile
  const uint32_t bo = ok ? u.slane + 256 * seg : kNoRow;
#pragma unroll
  for (int t = 0; t < TT; ++t) c.b[t] = __builtin_amdgcn_raw_buffer_load_b32(u.ws, (int)bo, (int)(u.ssoff + t * u.sstride), 0);
  if constexpr (ALDS)
    c.a = ok && u.aslane != kNoRow ? lds32(u.aslane - g + 16 * seg + 4 * g) : 0u;
  else
    c.a = bload32a<AUX>(u.as, ok ? u.aslane - g + 16 * seg + 4 * g : kNoRow, 0);
}

template <int TT>
__device__ __forceinline__ void transpose_codes4(Codes4<TT>& c, int g) {
#pragma unroll
  for (int t = 0; t < TT; ++t) c.b[t] = transpose4_groups(c.b[t], g);
  c.a = transpose4_groups(c.a, g);
}

template <int TT, int AUX, bool ALDS>
__device__ __forceinline__ void load_pair4(Pair4<TT>& f, const UnitOps& u, int st, int j) {
  const bool ok0 = st < u.nsteps, ok1 = st + 1 < u.nsteps;
  const uint32_t wo = (j < 8 ? ok0 : ok1) ? u.wlane + (uint32_t)st * 64 : kNoRow;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    f.x[t] = bload16_nt(u.w, wo, u.wsoff + t * u.tstride);
    f.y[t] = bload16_nt(u.w, wo, u.wsoff + t * u.tstride + u.row8);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if constexpr (ALDS) {
      const bool ar = (q ? ok1 : ok0) && u.alane != kNoRow;
      const uint32_t ao = u.alane + (uint32_t)(st + q) * 128;
      f.alo[q] = ar ? lds16(ao) : u32x4{0u, 0u, 0u, 0u};
      f.ahi[q] = ar ? lds16(ao + 64) : u32x4{0u, 0u, 0u, 0u};
    } else {
      const uint32_t ao = (q ? ok1 : ok0) ? u.alane + (uint32_t)(st + q) * 128 : kNoRow;
      f.alo[q] = bload16a<AUX>(u.a, ao, 0);
      f.ahi[q] = bload16a<AUX>(u.a, ao + 64, 0);
    }
  }
}

// Steps 2P and 2P + 1 of the segment (P: the pair's index in it).
template <int TT, int P>
__device__ __forceinline__ void mma_pair4(v4f (&acc)[TT], const Pair4<TT>& f, const Codes4<TT>& c) {
  const v8i a0 = join(f.alo[0], f.ahi[0]), a1 = join(f.alo[1], f.ahi[1]);
  const int sa0 = (int)((c.a >> (16 * P)) & 0xFF), sa1 = (int)((c.a >> (16 * P + 8)) & 0xFF);
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    u32x4 lo, hi;
    lines_to_mfma(f.x[t], f.y[t], lo, hi);
    acc[t] = mfma_e4m3_e2m1_sel<2 * P>(a0, lo, acc[t], sa0, c.b[t]);
    acc[t] = mfma_e4m3_e2m1_sel<2 * P + 1>(a1, hi, acc[t], sa1, c.b[t]);
  }
}

// One segment's sums for E2M1 weights: both line pairs (2 K steps each) and
// the codes loaded before the first MFMA; each tile's MFMAs run in K order.
template <int TT, int AUX, bool ALDS>
__device__ __forceinline__ void segment_sum_fp4(v4f (&acc)[TT], const UnitOps& u, int seg, int g, int j) {
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  Codes4<TT> c;
  Pair4<TT> f0, f1;
  load_codes4<TT, AUX, ALDS>(c, u, seg, g);
  load_pair4<TT, AUX, ALDS>(f0, u, seg * kSegSteps, j);
  load_pair4<TT, AUX, ALDS>(f1, u, seg * kSegSteps + 2, j);
  __builtin_amdgcn_sched_barrier(0);
  transpose_codes4<TT>(c, g);
  mma_pair4<TT, 0>(acc, f0, c);
  mma_pair4<TT, 1>(acc, f1, c);
  __builtin_amdgcn_sched_barrier(0);
}

// E4M3 weights: the segment sums of [s0, s1) added in segment order.  BSO:
// K steps per load burst (0: 2 for 8-tile units, else the whole segment).
template <int TT, int AUX, bool ALDS, int SEG, int BSO>
__device__ __forceinline__ void unit_sums_e4m3(v4f (&tot)[TT], const UnitOps& ops, int s0, int s1) {
  constexpr int BS = BSO ? BSO : TT >= 8 ? 2 : SEG;  // K steps per load burst
  segment_sum<TT, BS, AUX, ALDS, SEG>(tot, ops, s0);
  for (int sg = s0 + 1; sg < s1; ++sg) {
    v4f p[TT];
    segment_sum<TT, BS, AUX, ALDS, SEG>(p, ops, sg);
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) tot[t][q] = tot[t][q] + p[t][q];
  }
}

// The unit's sums over its segments [s0, s1), added in segment order; each
// segment's sum starts from zero.  BSO: the E4M3 load burst (K steps; 0: by
// tile count).  The burst only sets how many loads are in flight: each
// tile's MFMAs run in K order whatever it is, so the sums do not change.
template <int TT, int AUX, bool ALDS = false, int BSO = 0>
__device__ __forceinline__ void unit_sums(v4f (&tot)[TT], const UnitOps& ops, int s0, int s1, int g, int j) {
  if (ops.fp4) {
    segment_sum_fp4<TT, AUX, ALDS>(tot, ops, s0, g, j);
    for (int sg = s0 + 1; sg < s1; ++sg) {
      v4f p[TT];
      segment_sum_fp4<TT, AUX, ALDS>(p, ops, sg, g, j);
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) tot[t][q] = tot[t][q] + p[t][q];
    }
  } else if (ops.seg == 2) {
    unit_sums_e4m3<TT, AUX, ALDS, 2, BSO>(tot, ops, s0, s1);
  } else {
    unit_sums_e4m3<TT, AUX, ALDS, kSegSteps, BSO>(tot, ops, s0, s1);
  }
}

// Units of one run, in order: the shared slots' units, then the routed ones;
// inside a slot tile-group-major, segment-minor (split mode) or one per tile
// group.
struct UnitMap {
  int nS, nvs, per_s, per_r, split;
  int nseg_s, nseg_r;
  uint32_t total;
};

template <bool W13, int TT>
__device__ __forceinline__ UnitMap unit_map_n(const LayerDims& d, int nvs, int nS, int split) {
  UnitMap um;
  um.nvs = nvs;
  um.nS = nS;
  um.split = split;
  const Geo gs = geo<W13>(d, true), gr = geo<W13>(d, false);
  um.nseg_s = gs.nseg;
  um.nseg_r = gr.nseg;
  um.per_s = gs.tiles / TT * (split ? gs.nseg : 1);
  um.per_r = gr.tiles / TT * (split ? gr.nseg : 1);
  um.total = (uint32_t)(um.nS * um.per_s + (um.nvs - um.nS) * um.per_r);
  return um;
}

template <bool W13, int TT>
__device__ __forceinline__ UnitMap unit_map(const LayerDims& d, const Scratch& s, int split) {
  return unit_map_n<W13, TT>(d, s.header[0], s.header[1], split);
}

// unit -> (slot, tile group, first segment, end segment)
__device__ __forceinline__ void unit_decode(const UnitMap& um, uint32_t u, int& v, int& tg, int& s0, int& s1) {
  int rem, nseg;
  const uint32_t shared_units = (uint32_t)(um.nS * um.per_s);
  if (u < shared_units) {
    v = (int)(u / (uint32_t)um.per_s);
    rem = (int)u - v * um.per_s;
    nseg = um.nseg_s;
  } else {
    const uint32_t u2 = u - shared_units;
    const int vr = (int)(u2 / (uint32_t)um.per_r);
    v = um.nS + vr;
    rem = (int)u2 - vr * um.per_r;
    nseg = um.nseg_r;
  }
  if (um.split) {
    tg = rem / nseg;
    s0 = rem - tg * nseg;
    s1 = s0 + 1;
  } else {
    tg = rem;
    s0 = 0;
    s1 = nseg;
  }
}

// The unit of a block's turn i: the units are dealt in rows of B, one per
// block, the order of the blocks reversed every other row.  Consecutive
// units are consecutive K segments of a tile group, so without the reversal
// a block (and an XCD, which runs every eighth block) would only ever see
// one parity of segment: the XCDs that read the odd 512-byte segments of
// the rows took 12% longer.
__device__ __forceinline__ uint32_t unit_turn(uint32_t i, uint32_t B, uint32_t b) {
  return i * B + ((i & 1u) ? B - 1u - b : b);
}

// The routed slots of a w13 launch that routes in its first blocks, built in
// the block's LDS by the first wave that needs them (the others wait for
// that wave): the wave reads the pick box until every pick of the step
// carries the tag, then sorts the picks into the plan's rows (small_rows:
// the same rows and slots as the router's plan).  On a timeout the status
// word is set and no routed slot is staged.
// s_out (may be null): also each routed row's w2 output row, its pair.
// Returns the slots the calling wave may use: the staged ones, or only the
// nS shared ones when it gave up waiting for the staging wave (whose LDS
// writes it then must not read).  The count is the same in every lane of
// the wave; it is returned (and taken by the callers) through
// readfirstlane, since the unit map and the deal derived from it otherwise
// compile to per-lane arithmetic and branches.
__device__ int stage_plan(const LayerDims& d, const Scratch& s, int4* s_vs, int* s_tok, int nS, int P, int vs_cap,
                          int* s_plan, int* s_nvs, int lane, int* s_out = nullptr) {
  int st = 0;
  if (lane == 0) st = atomicCAS(s_plan, 0, 1);
  st = __builtin_amdgcn_readfirstlane(st);
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  if (st == 0) {
    uint32_t w = 0;
    bool in = false;
    while (true) {
      w = lane < P ? load_coherent(s.pick_box + lane) : kBoxTag;
      if (__ballot(!(w & kBoxTag)) == 0ull) {
        in = true;
        break;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > s.wait_ticks) {
        if (lane == 0) flag_status(s.status, kStatusRouteWait);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    const int n = in ? P : 0;
    const SmallRows q = small_rows((int)(w & 0x3FFu), n, d.K, lane);
    const int nR = min(q.nR, vs_cap - nS);
    if (q.valid) s_tok[lane] = q.t;
    if (q.valid && s_out) s_out[lane] = q.p;
    if (q.first && q.ri < nR) s_vs[nS + q.ri] = make_int4(q.e, lane, q.cnt, 0);
    if (lane == 0) *s_nvs = nS + nR;
    wait_memory();  // the LDS writes are done
    if (lane == 0) __hip_atomic_store(s_plan, 2, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    return __builtin_amdgcn_readfirstlane(nS + nR);
  }
  while (__hip_atomic_load(s_plan, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != 2) {
    __builtin_amdgcn_s_sleep(1);
    if (__builtin_amdgcn_s_memrealtime() - t0 > 2 * s.wait_ticks) {
      if (lane == 0) flag_status(s.status, kStatusRouteWait);
      return nS;
    }
  }
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(s_nvs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}

// The seam of the w13 launch that routes (m <= kRouteRows rows, H <= 8192),
// run by all eight waves of the block with the seam launch's thread mapping
// (8 columns a thread, chunks of kSeamChunk) and order of every sum, so its
// bits are that launch's:
//   - the rows' RMSNorm and MXFP8 into the block's LDS (values at x8o, codes
//     at xso): the A operand of the block's w13 units;
//   - the router logits of experts b and b + G for every row (b: the block,
//     G: the blocks of the launch), stored tagged into the logit box;
//   - block 0 also stores the normed rows and the MXFP8 (s.normed, s.x8,
//     s.x8s) for inspection.
// Every thread of the block calls it; the LDS rows are complete when the
// barrier inside has passed.
__device__ void seam_rows(const LayerDims& d, int m, const Inputs& in, const Scratch& s, uint32_t x8o,
                          uint32_t xso) {
  constexpr int CPT = 2, EB = 2;  // H <= 2 kSeamChunk
  __shared__ double red_ss[kRouteRows][kSeamWaves];
  __shared__ double red_lg[kRouteRows][EB][kSeamWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool seam = tid < kSeamThreads;
  const int H = d.H, E = d.E, G = gridDim.x, b = blockIdx.x;
  const bool taps = b == 0;
  int col[CPT];
  bool live[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    col[q] = 8 * tid + kSeamChunk * q;
    live[q] = seam && col[q] < H;
  }
  // every load at once: the rows, the norm weight, the block's gate rows
  u32x4 xv[kRouteRows][CPT], wv[CPT], gv[EB][CPT];
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int t = 0; t < kRouteRows; ++t)
#pragma unroll
    for (int q = 0; q < CPT; ++q)
      xv[t][q] = (t < m && live[q]) ? ld16(reinterpret_cast<const uint8_t*>(in.x + (size_t)t * H + col[q])) : zero;
#pragma unroll
  for (int q = 0; q < CPT; ++q) wv[q] = live[q] ? ld16(reinterpret_cast<const uint8_t*>(in.norm_w + col[q])) : zero;
#pragma unroll
  for (int k = 0; k < EB; ++k) {
    const int e = b + k * G;
#pragma unroll
    for (int q = 0; q < CPT; ++q)
      gv[k][q] = (e < E && live[q]) ? ld16(reinterpret_cast<const uint8_t*>(in.gate_w + (size_t)e * H + col[q])) : zero;
  }
  // sums of squares in double, lanes then waves in a fixed order
#pragma unroll
  for (int t = 0; t < kRouteRows; ++t) {
    if (t >= m) break;
    double ss = 0.0;
#pragma unroll
    for (int q = 0; q < CPT; ++q)
      if (live[q]) ss = add_squares8(ss, xv[t][q]);
    ss = wave_sum(ss);
    if (seam && lane == 0) red_ss[t][wave] = ss;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kRouteRows; ++t) {
    if (t >= m) break;
    double sst = red_ss[t][0];
#pragma unroll
    for (int w = 1; w < kSeamWaves; ++w) sst += red_ss[t][w];
    const float r = (float)(1.0 / sqrt(sst / (double)H + (double)d.eps));
    double acc[EB];
#pragma unroll
    for (int k = 0; k < EB; ++k) acc[k] = 0.0;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      float y[8];
      uint32_t yb[8];
      if (live[q]) {
        norm8(xv[t][q], wv[q], r, y, yb);
#pragma unroll
        for (int k = 0; k < EB; ++k)
          if (b + k * G < E) acc[k] = add_logit8(acc[k], y, gv[k][q]);
      } else {
#pragma unroll
        for (int z = 0; z < 8; ++z) {
          y[z] = 0.0f;
          yb[z] = 0u;
        }
      }
      u32x2 qv;
      const int code = mx8(y, qv);
      if (live[q]) {
        *reinterpret_cast<u32x2*>(dyn_lds + x8o + (uint32_t)(t * H + col[q])) = qv;
        if ((lane & 3) == 0) dyn_lds[xso + (uint32_t)(t * (H / 32) + col[q] / 32)] = (uint8_t)code;
        if (taps) {
          u32x4 nv;
#pragma unroll
          for (int z = 0; z < 4; ++z) nv[z] = yb[2 * z] | (yb[2 * z + 1] << 16);
          *reinterpret_cast<u32x4*>(s.normed + (size_t)t * H + col[q]) = nv;
          *reinterpret_cast<u32x2*>(s.x8 + (size_t)t * H + col[q]) = qv;
          if ((lane & 3) == 0) s.x8s[(size_t)t * (H / 32) + col[q] / 32] = (uint8_t)code;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < EB; ++k) {
      const double tot = wave_sum(acc[k]);
      if (seam && lane == 0) red_lg[t][k][wave] = tot;
    }
  }
  __syncthreads();
  if (tid < m * EB) {
    const int t = tid / EB, k = tid % EB, e = b + k * G;
    if (e < E) {
      double v = red_lg[t][k][0];
#pragma unroll
      for (int w = 1; w < kSeamWaves; ++w) v += red_lg[t][k][w];
      uint64_t w = (uint64_t)__double_as_longlong(v) ^ kLogitTag;
      if (w == 0ull) w = kLogitTag;  // (-0 is not a sum from +0; kept as +0 all the same)
      __hip_atomic_store(&s.logit_box[(size_t)t * E + e], w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The GEMM, one block of NW waves per CU.  Block b of B takes one unit of
// every row of B units (unit_turn), so every CU streams the same bytes and
// gets its part of every slot; its waves take the block's units from a
// counter in LDS, so a slow wave does not hold the CU back.  Lane (g, j) of a unit ends with rows
// 4g..4g+3 of the slot and weight rows col0 + 16 t + j; rows past the slot's
// c are not stored.  Split units store their segment sums in plane s0 of
// `part`, whole units the tiles' totals in plane 0.  Part planes are
// [R][width] fp32, R = m (k + 1).
// One unit of the GEMM: TT tiles of tile group tgroup (in units of TT
// tiles) of a slot over segments [s0, s1).  w13 sums go to the slot's rows,
// w2 sums to the rows' output rows (plane s0 in split mode, else plane 0).
template <bool W13, int TT, bool ROUTE>
__device__ __forceinline__ void run_unit(const int4& slot, int tgroup, int s0, int s1, bool split, const LayerDims& d,
                                         const Inputs& in, const Scratch& s, const int* s_tok, int m, int R, int g,
                                         int j, uint32_t x8o, uint32_t xso, float* part, size_t plane, int width) {
  const UnitOps ops = unit_ops<W13, TT, ROUTE>(slot, tgroup, d, in, s, s_tok, m, R, g, j, x8o, xso);
  v4f tot[TT];
  // the launch that routes loads 2 K steps (16 KB) a burst: its blocks' pick
  // polls then wait behind less (m = 1: 4-step bursts 63.4-63.7 us against
  // 63.1-63.2, 1-step bursts slower still)
  unit_sums<TT, 0, ROUTE, ROUTE ? 2 : 0>(tot, ops, s0, s1, g, j);
  float* dst = part + (size_t)(split ? s0 : 0) * plane + ops.col0 + j;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (4 * g + q < ops.c) {
      const int r = ops.row0 + 4 * g + q;
      const size_t orow = (size_t)(W13 ? r : s_tok[r]);
#pragma unroll
      for (int t = 0; t < TT; ++t) dst[orow * width + 16 * t] = tot[t][q];
    }
  }
}

// The first turn dealt as half units: the units of a run's last, partial
// row of B (fewer than B) are cut in two halves of TT / 2 tiles (the same
// sums: tiles are independent), dealt one per block, so every block streams
// about the same bytes (w2 at 48 rows: 326 -> 320 us).  ~0u: no halves.
__device__ __forceinline__ uint32_t half_row(uint32_t total, uint32_t B, int TT) {
  return (TT >= 4 && total % B != 0) ? total / B : 0xFFFFFFFFu;
}

template <bool W13, int TT, int NW, bool ROUTE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4)))
void gemm_kernel(LayerDims d, Inputs in, Scratch s, int m, int split, int vs_cap) {
  unsigned char* lds_raw = dyn_lds;
  __shared__ uint32_t s_next;
  __shared__ int s_plan, s_nvs;  // ROUTE: the plan's staging state (0, 1, 2) and slot count
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  uint64_t* tl = W13 ? s.tl_w13 : s.tl_w2;
  stamp(tl, kTlPoints, 0);
  const int R = m * d.K + m;
  const int P = m * d.K;
  // after the slots and the row map: ROUTE, the MXFP8 rows; other w13
  // launches, the LDS of the plan they build
  const uint32_t x8o = ((uint32_t)vs_cap * 16 + (uint32_t)R * 4 + 15u) & ~15u;
  const uint32_t xso = x8o + (uint32_t)(m * d.H);
  if constexpr (ROUTE) {
    static_assert(NW * 64 == kSeamThreads, "the seam's thread mapping takes the whole block");
    seam_rows(d, m, in, s, x8o, xso);
    stamp(tl, kTlPoints, 2);
    // blocks [0, m) route the m tokens from the logit box and store their
    // picks in the pick box; the last of them builds the plan for the
    // launches after this one
    if ((int)blockIdx.x < m) {
      __shared__ RouteLds L;
      (void)route_block<1>(d, m, blockIdx.x, m, in.bias, s, L, s.pick_box, s.logit_box);
      return;
    }
  }
  int4* s_vs = reinterpret_cast<int4*>(lds_raw);
  int* s_tok = reinterpret_cast<int*>(s_vs + vs_cap);  // w13: token of a row; w2: its output row
  UnitMap um;
  if constexpr (ROUTE) {
    // until the picks are in: the shared expert's slots and rows, which do
    // not depend on the routing
    const int nS = (m + kTokTile - 1) / kTokTile;
    um = unit_map_n<W13, TT>(d, nS, nS, split);
    for (int v = tid; v < nS; v += NW * 64) {
      const int rows = m - v * kTokTile;
      s_vs[v] = make_int4(-1, P + v * kTokTile, rows < kTokTile ? rows : kTokTile, 0);
    }
    for (int t = tid; t < m; t += NW * 64) s_tok[P + t] = t;
    if (tid == 0) s_plan = 0;
  } else if constexpr (W13) {
    // the plan, from the picks the route launch stored (after the slots and
    // the row map in the LDS); block 0 also stores it for the w2 launch and
    // the taps
    const int nvs = plan_block<NW>(d, m, s, s_vs, s_tok, reinterpret_cast<uint32_t*>(lds_raw + x8o), blockIdx.x == 0);
    um = unit_map_n<W13, TT>(d, nvs, (m + kTokTile - 1) / kTokTile, split);
  } else {
    // the whole slot table (vs_cap entries, allocated for the plan's widest
    // step) beside the header's load, instead of after it
    for (int i = tid; i < vs_cap; i += NW * 64) s_vs[i] = s.vslots[i];
    um = unit_map<W13, TT>(d, s, split);
    for (int i = tid; i < R; i += NW * 64) s_tok[i] = s.row_out[i];
  }
  if (tid == 0) s_next = 0;
  __syncthreads();

  const int width = W13 ? 2 * d.Imax : d.H;
  float* part = W13 ? s.part13 : s.part2;
  const size_t plane = (size_t)R * width;
  // the block's turns i take unit unit_turn(i): units of one slot (costlier
  // for slots with more rows) spread over every CU (the routing blocks take
  // none)
  const uint32_t nroute = ROUTE ? (uint32_t)m : 0u;
  const uint32_t B = gridDim.x - nroute, b = blockIdx.x - nroute;
  bool planned = !ROUTE;
  // the launch that routes keeps whole units to the end: a second unit
  // body there spilled registers and slowed it more than the tail gained
  uint32_t hrow = ROUTE ? 0xFFFFFFFFu : half_row(um.total, B, TT);
  // first unit by wave index, the rest from the block's counter; the next
  // index is fetched while the current unit streams
  uint32_t i = wave;
  while (true) {
    uint32_t u;
    int half = -1;
    if constexpr (ROUTE) {
      u = unit_turn(i, B, b);
      if (u >= um.total) {
        // past the shared expert's units: the routed ones need the picks
        if (planned) break;
        const int nvs = __builtin_amdgcn_readfirstlane(stage_plan(d, s, s_vs, s_tok, um.nS, P, vs_cap, &s_plan, &s_nvs, lane));
        um = unit_map_n<W13, TT>(d, nvs, um.nS, split);
        planned = true;
        if (u >= um.total) break;  // the last turn has no unit for this block
      }
    } else if (i < hrow) {
      u = unit_turn(i, B, b);
      if (u >= um.total) break;
    } else {
      const uint32_t h = unit_turn(i - hrow, B, b);
      if (h >= 2u * (um.total - hrow * B)) break;
      u = hrow * B + h / 2u;
      half = (int)(h & 1u);
    }
    uint32_t nx = 0;
    if (lane == 0) nx = __hip_atomic_fetch_add(&s_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    int v, tg, s0, s1;
    unit_decode(um, u, v, tg, s0, s1);
    if constexpr (TT >= 4 && !ROUTE) {
      if (half >= 0)
        run_unit<W13, TT / 2, ROUTE>(s_vs[v], 2 * tg + half, s0, s1, um.split, d, in, s, s_tok, m, R, g, j, x8o,
                                     xso, part, plane, width);
      else
        run_unit<W13, TT, ROUTE>(s_vs[v], tg, s0, s1, um.split, d, in, s, s_tok, m, R, g, j, x8o, xso, part, plane,
                                 width);
    } else {
      run_unit<W13, TT, ROUTE>(s_vs[v], tg, s0, s1, um.split, d, in, s, s_tok, m, R, g, j, x8o, xso, part, plane,
                               width);
    }
    i = NW + (uint32_t)__builtin_amdgcn_readfirstlane((int)nx);
  }
  stamp_wave(tl, kTlPoints, 3 + (wave & 3));
  __syncthreads();
  stamp(tl, kTlPoints, 1);
}

// a = SiLU(gate) * up of row r, column col (one lane each, 32 consecutive
// columns in 32 consecutive lanes), and its MXFP8: the code of the 32
// columns' amax, the byte of a scaled by 2^(127 - code).
__device__ __forceinline__ void act_store(const LayerDims& d, const Scratch& s, int r, int col, float hg, float hu) {
  const float a = hg / (1.0f + __expf(-hg)) * hu;
  const float amax = group_max(fabsf(a), 32);
  const int code = e8m0_code(amax);
  s.a8[(size_t)r * d.Imax + col] = (uint8_t)(fp8x2(a * mx_mul(code), 0.0f) & 0xFF);
  if ((col & 31) == 0) s.a8s[(size_t)r * (d.Imax / 32) + col / 32] = (uint8_t)code;
}

// SiLU(gate) * up of row r (blockIdx.y), columns blockIdx.x * 256 + tid, and
// the MXFP8 of each 32 columns (one lane group of 32 per code).  The NSEG
// bound makes every load unconditional (planes past the run's count are read
// from its last plane and not added), so they are all in flight at once.
template <int NSEG>
__global__ __launch_bounds__(kThreads) void act_kernel(LayerDims d, Scratch s, int m, int split) {
  const int r = blockIdx.y, c = blockIdx.x * kThreads + threadIdx.x;
  const int P = m * d.K;
  const int Kv = r < P ? d.I : d.Is;
  stamp(s.tl_act, kTlPoints, 0);
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    // the boxes of a w13 launch that routes start the next run at zero
    for (int w = threadIdx.x; w < kPickBox; w += kThreads) s.pick_box[w] = 0u;
    if (s.logit_box)
      for (int w = threadIdx.x; w < kRouteRows * d.E; w += kThreads) s.logit_box[w] = 0ull;
  }
  if (c >= Kv) return;  // whole groups of 32 (Kv is a multiple of 128)
  const int nseg = split ? (d.H / 128 + kSegSteps - 1) / kSegSteps : 1;
  const size_t plane = (size_t)(m * d.K + m) * 2 * d.Imax;
  const float* p = s.part13 + (size_t)r * 2 * d.Imax;
  float vg[NSEG], vu[NSEG];
#pragma unroll
  for (int sg = 0; sg < NSEG; ++sg) {
    const size_t o = (size_t)(sg < nseg ? sg : nseg - 1) * plane;
    vg[sg] = p[o + c];
    vu[sg] = p[o + Kv + c];
  }
  float hg = vg[0], hu = vu[0];
#pragma unroll
  for (int sg = 1; sg < NSEG; ++sg) {
    hg = sg < nseg ? hg + vg[sg] : hg;
    hu = sg < nseg ? hu + vu[sg] : hu;
  }
  act_store(d, s, r, c, hg, hu);
  stamp(s.tl_act, kTlPoints, 1);
}

// out[t, n] (t = blockIdx.y, one column per lane): the routed rows' y
// weighted in selection order, then the shared row, in fp32; one rounding to
// bf16.  The w2 sums of pick (t, j) sit in row t k + j, the shared row's in
// row m k + t, so every load is issued at once.  Narrow blocks spread the
// reads over many CUs.
constexpr int kCombineThreads = 64;

template <int NSEG>
__device__ __forceinline__ float row_sum(const float* p, size_t plane, int nseg) {
  float v[NSEG];
#pragma unroll
  for (int sg = 0; sg < NSEG; ++sg) v[sg] = p[(size_t)(sg < nseg ? sg : nseg - 1) * plane];
  float y = v[0];
#pragma unroll
  for (int sg = 1; sg < NSEG; ++sg) y = sg < nseg ? y + v[sg] : y;
  return y;
}

// NSEG bounds the run's segment counts; every load is unconditional (picks
// past k and planes past the count re-read valid addresses and are not
// added), so a lane's loads are all in flight at once.
// clear: also zero the hand-off words of the persistent launch (from word 1
// of the sync region: XCC ids, ready words, act counts, the boxes) for the
// next step; word 0, the route blocks' arrival counter, resets itself.
template <int NSEG>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(LayerDims d, Inputs in, Scratch s, int m,
                                                                  int split, int clear) {
  const int t = blockIdx.y, n = blockIdx.x * kCombineThreads + threadIdx.x;
  stamp(s.tl_combine, kTlPoints, 0);
  if (clear) {
    const uint32_t nthr = gridDim.x * gridDim.y * kCombineThreads;
    for (uint32_t w = 1 + (blockIdx.y * gridDim.x + blockIdx.x) * kCombineThreads + threadIdx.x;
         w < (uint32_t)s.nsync; w += nthr)
      s.sync[w] = 0u;
  }
  if (n >= d.H) return;
  const int P = m * d.K;
  const int seg_r = w2_seg_steps(d, d.I, d.rfmt == MOE_DECODE_ROUTED_MXFP4), seg_s = w2_seg_steps(d, d.Is, false);
  const int nseg_r = split ? (d.I / 128 + seg_r - 1) / seg_r : 1;
  const int nseg_s = split ? (d.Is / 128 + seg_s - 1) / seg_s : 1;
  const size_t plane = (size_t)(m * d.K + m) * d.H;
  const float ysh = row_sum<NSEG>(s.part2 + (size_t)(P + t) * d.H + n, plane, nseg_s);
  float acc = 0.0f;
  for (int k0 = 0; k0 < d.K; k0 += 8) {
    float w[8], y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = t * d.K + (k0 + i < d.K ? k0 + i : d.K - 1);
      w[i] = s.wts[p];
      y[i] = row_sum<NSEG>(s.part2 + (size_t)p * d.H + n, plane, nseg_r);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = k0 + i < d.K ? fmaf(w[i], y[i], acc) : acc;
  }
  acc = acc + ysh;
  in.out[(size_t)t * d.H + n] = (uint16_t)f32_to_bf16(acc);
  stamp(s.tl_combine, kTlPoints, 1);
}

// Tiles per unit and waves per block (one block per CU) of each GEMM and
// mode.  More tiles per unit share one activation fragment among more weight
// tiles and keep more weight bytes in flight per wave; fewer tiles give more
// units to balance at small m.  Each tile's sums are the same whichever
// variant runs it.  Whole-mode w13 units take 4 tiles: a block's 25-26
// units of 8 tiles (655 KB each at H = 5120) left one wave streaming the
// last unit alone for up to 40 us after its block's other waves ended.
// Split-mode w2 units take 8 tiles where a w2 segment is 2 K steps, so a
// unit still streams 32 KB.
constexpr int kTT13 = 4;       // w13 units, both modes
constexpr int kTT2Whole = 8;   // whole-mode w2 units
constexpr int kTT2Split = 4;   // split-mode w2 units over 4-step segments
constexpr int kGemmWaves = 8;  // waves per block of either GEMM
// K steps per load burst of the persistent launch's units (w13, w2): 16 KB
// a wave for w13 (as in the w13 launch that routes, whose pick polls then
// queue behind less), a whole 256-column w2 slice for w2.
constexpr int kXcdBurst13 = 2;
constexpr int kXcdBurst2 = 2;

// ===========================================================================
// The persistent launch of a step of at most kRouteRows tokens: the seam,
// the router, w13, SiLU * up and w2 in one launch of one block per CU, cut by
// XCD.  The dispatcher deals a launch's blocks to the XCDs round-robin
// (from where the previous launch left off), so the blocks with index x mod
// kXcds share one XCD: the plan checks that on the device, and each block
// checks it against the others at its end.  Those blocks take slice x of
// every active expert's intermediate: gate rows [x S, (x + 1) S) and up rows
// [Kv + x S, ...) of w13 (S = Kv / kXcds), and the same S columns of w2.
// So every hand-off -- the w13 sums to SiLU * up, the a8 to w2 -- stays
// inside one XCD's L2, which every CU of the XCD shares.  Nothing crosses
// XCDs until the launch ends: the combine launch adds the slices' w2 sums
// (plane x holds slice x) in slice order, which is the w2 segment order of
// every other step width (w2 segments are S = 256 columns here).
//
// Each XCD runs three phases, its blocks meeting at a barrier between them
// (an arrival count performed in the XCD's L2):
//   1. w13: the shared expert's units (tile groups of 64 rows in the slice,
//      times the H segments), then, once the picks are in, every routed
//      slot's, dealt over the XCD's blocks (the m route blocks, rank 0 of
//      XCDs 0..m-1, take none);
//   2. SiLU * up: the slice's act groups (slot, 64 columns), one a wave,
//      with the act launch's arithmetic on the summed planes;
//   3. w2: the shared expert's units (tile groups of 128 output rows over
//      the slice), then every routed slot's.
// The sums and a8 (values and codes) are stored and completed before a
// block arrives, and read after the barrier by loads that reach the L2
// (sc0) from CUs that have not read those lines before in the launch.
// Each barrier's count sits in a cache line of its own.  Per-slot counts
// that let w2 units start before the whole w13 phase ended were measured
// slower: each hand-off then queued behind the weight stream.
// ===========================================================================

__device__ __forceinline__ float ld_l2(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kScL2));
}

// The a8 of act group q (64 columns, lane = column) of slot `slot` from the
// w13 sums of its nseg planes, every row of the slot.
__device__ void act_group(const LayerDims& d, const Scratch& s, int m, const int4& slot, int q, int nseg,
                          int lane) {
  const int Kv = slot.x < 0 ? d.Is : d.I;
  const uint32_t width = 2u * (uint32_t)d.Imax;
  const uint32_t plane = (uint32_t)(m * d.K + m) * width;
  const rsrc_t pr = make_rsrc(s.part13, (uint32_t)nseg * plane * 4u);
  const int col = kActCols * q + lane;
  for (int i = 0; i < slot.z; ++i) {
    const uint32_t o = ((uint32_t)(slot.y + i) * width + (uint32_t)col) * 4u;
    float vg[16], vu[16];
    float hg = 0.0f, hu = 0.0f;
    for (int s0 = 0; s0 < nseg; s0 += 16) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int sg = s0 + k < nseg ? s0 + k : nseg - 1;
        vg[k] = ld_l2(pr, o + (uint32_t)sg * plane * 4u);
        vu[k] = ld_l2(pr, o + ((uint32_t)sg * plane + (uint32_t)Kv) * 4u);
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (s0 + k < nseg) {
          hg = s0 + k == 0 ? vg[k] : hg + vg[k];
          hu = s0 + k == 0 ? vu[k] : hu + vu[k];
        }
      }
    }
    act_store(d, s, slot.y + i, col, hg, hu);
  }
}

// The count in an arrival word, read in the XCD's L2.  A load, even at
// workgroup scope, may be served by this CU's own cache, which would keep
// the first value it saw; an atomic is performed in the L2.  An atomic that
// changes nothing (adding 0) is compiled into a load, so the read sets bit
// 31, which the counts never reach, and masks it off.  The combine launch
// zeroes the words for the next step.
constexpr uint32_t kPeekBit = 0x80000000u;
__device__ __forceinline__ uint32_t peek_l2(uint32_t* p) {
  return __hip_atomic_fetch_or(p, kPeekBit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) & ~kPeekBit;
}

// Barrier of the `blocks` blocks of one XCD on arrival word w: every wave's
// stores completed, the block counted once, and wave 0 reads the word until
// it holds every block.  A wait past s.wait_ticks sets the status word (the
// block then goes on).  Called by every thread of the block.
__device__ void xcd_barrier(uint32_t* w, uint32_t blocks, const Scratch& s, int tid) {
  wait_memory();
  __syncthreads();
  if (tid < 64) {
    if (tid == 0) (void)__hip_atomic_fetch_add(w, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (true) {
      uint32_t c = 0;
      if (tid == 0) c = peek_l2(w);
      if (__builtin_amdgcn_readfirstlane((int)c) >= (int)blocks) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > s.wait_ticks) {
        if (tid == 0) flag_status(s.status, kStatusA8Wait);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4)))
void xcd_kernel(LayerDims d, Inputs in, Scratch s, int m, int vs_cap) {
  constexpr int TT13 = kTT13, TT2 = 8;
  unsigned char* lds_raw = dyn_lds;
  __shared__ uint32_t s_next;
  __shared__ int s_plan, s_nvs;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  stamp(s.tl_experts, kTlPoints, 0);
  const int b = blockIdx.x, x = b % kXcds, rank = b / kXcds;
  const int R = m * d.K + m, P = m * d.K;
  // LDS: the slots, row -> token, row -> w2 output row, then the MXFP8 rows
  const uint32_t x8o = ((uint32_t)vs_cap * 16 + (uint32_t)R * 8 + 15u) & ~15u;
  const uint32_t xso = x8o + (uint32_t)(m * d.H);
  seam_rows(d, m, in, s, x8o, xso);
  stamp(s.tl_experts, kTlPoints, 2);
  if (b < m) {
    __shared__ RouteLds L;
    (void)route_block<1>(d, m, b, m, in.bias, s, L, s.pick_box, s.logit_box);
    return;
  }
  int4* s_vs = reinterpret_cast<int4*>(lds_raw);
  int* s_tok = reinterpret_cast<int*>(s_vs + vs_cap);
  int* s_out = s_tok + R;
  constexpr int nS = 1;  // m <= kRouteRows rows: one shared slot
  if (tid == 0) {
    s_vs[0] = make_int4(-1, P, m, 0);
    s_plan = 0;
    s_next = 0;
  }
  if (tid < m) {
    s_tok[P + tid] = tid;
    s_out[P + tid] = P + tid;
  }
  __syncthreads();

  // this block's share of its XCD's units
  const int r0 = x < m ? 1 : 0;
  const uint32_t Bw = (uint32_t)(gridDim.x / kXcds - r0), rw = (uint32_t)(rank - r0);
  const int Ss = d.Is / kXcds, Sr = d.I / kXcds;
  const int nseg13 = (d.H / 128 + kSegSteps - 1) / kSegSteps;
  const uint32_t u13s = (uint32_t)(2 * Ss / 64 * nseg13), u13r = (uint32_t)(2 * Sr / 64 * nseg13);
  const uint32_t u2 = (uint32_t)(d.H / (16 * TT2));
  const uint32_t width13 = 2u * (uint32_t)d.Imax;
  const size_t plane13 = (size_t)R * width13, plane2 = (size_t)R * d.H;

  // phase 1, w13: the shared expert's turns, then (once the picks are in)
  // the routed slots' turns
  const uint32_t tA = (u13s + Bw - 1) / Bw;
  uint32_t nC = 0, tC = 0;
  int nvs = nS;
  bool planned = false;
  uint32_t i = wave;
  while (true) {
    uint32_t u, units;
    bool shared;
    if (i < tA) {
      u = unit_turn(i, Bw, rw), units = u13s, shared = true;
    } else {
      if (!planned) {
        nvs = __builtin_amdgcn_readfirstlane(
            stage_plan(d, s, s_vs, s_tok, nS, P, vs_cap, &s_plan, &s_nvs, lane, s_out));
        nC = (uint32_t)(nvs - nS) * u13r;
        tC = (nC + Bw - 1) / Bw;
        planned = true;
      }
      if (i >= tA + tC) break;
      u = unit_turn(i - tA, Bw, rw), units = nC, shared = false;
    }
    uint32_t nx = 0;
    if (lane == 0) nx = __hip_atomic_fetch_add(&s_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (u < units) {
      // slot, tile group in the slice (gate groups, then up groups), H segment
      const uint32_t per = shared ? u13s : u13r;
      const int v = shared ? 0 : nS + (int)(u / per);
      const uint32_t uu = u % per;
      const int tg = (int)(uu / (uint32_t)nseg13), seg = (int)(uu % (uint32_t)nseg13);
      const int S = shared ? Ss : Sr, Kv = shared ? d.Is : d.I;
      const int gps = S / 64;  // act groups (and gate tile groups) per slice
      const int q = x * gps + (tg % gps);
      const int tgroup = tg < gps ? q : (Kv / 64 + q);
      const UnitOps ops = unit_ops<true, TT13, true>(s_vs[v], tgroup, d, in, s, s_tok, m, R, g, j, x8o, xso);
      v4f tot[TT13];
      unit_sums<TT13, 0, true, kXcdBurst13>(tot, ops, seg, seg + 1, g, j);
      float* dst = s.part13 + (size_t)seg * plane13 + ops.col0 + j;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        if (4 * g + qq < ops.c) {
          const size_t r = (size_t)(ops.row0 + 4 * g + qq);
#pragma unroll
          for (int t = 0; t < TT13; ++t) dst[r * width13 + 16 * t] = tot[t][qq];
        }
      }
    }
    i = NW + (uint32_t)__builtin_amdgcn_readfirstlane((int)nx);
  }
  // (every wave leaves the loop through the routed turns, so it has read
  // the slot count)
  stamp(s.tl_experts, kTlPoints, 3);
  xcd_barrier(&s.sync[kXcdBarrierBase + x * kXcdBarrierStride], Bw, s, tid);

  // phase 2, SiLU * up: act group k of the slice (the shared slot's gps_s,
  // then gps_r per routed slot), one a wave
  const int gps_s = Ss / kActCols, gps_r = Sr / kActCols;
  const uint32_t nact = (uint32_t)(gps_s + (nvs - nS) * gps_r);
  for (uint32_t k = (uint32_t)wave * Bw + rw; k < nact; k += (uint32_t)NW * Bw) {
    const bool shared = k < (uint32_t)gps_s;
    const int v = shared ? 0 : nS + (int)((k - gps_s) / (uint32_t)gps_r);
    const int ql = shared ? (int)k : (int)((k - gps_s) % (uint32_t)gps_r);
    act_group(d, s, m, s_vs[v], x * (shared ? gps_s : gps_r) + ql, nseg13, lane);
  }
  if (tid == 0) s_next = 0;
  stamp(s.tl_experts, kTlPoints, 4);
  xcd_barrier(&s.sync[kXcdBarrierBase + (kXcds + x) * kXcdBarrierStride], Bw, s, tid);

  // phase 3, w2: slot, tile group of output rows, over the slice's K steps
  const uint32_t n2 = (uint32_t)nvs * u2, t2 = (n2 + Bw - 1) / Bw;
  i = wave;
  while (i < t2) {
    const uint32_t u = unit_turn(i, Bw, rw);
    uint32_t nx = 0;
    if (lane == 0) nx = __hip_atomic_fetch_add(&s_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (u < n2) {
      const int v = (int)(u / u2), tg = (int)(u % u2);
      const UnitOps ops = unit_ops<false, TT2>(s_vs[v], tg, d, in, s, s_out, m, R, g, j);
      v4f tot[TT2];
      unit_sums<TT2, kScL2, false, kXcdBurst2>(tot, ops, x, x + 1, g, j);
      float* dst = s.part2 + (size_t)x * plane2 + ops.col0 + j;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        if (4 * g + qq < ops.c) {
          const size_t orow = (size_t)s_out[ops.row0 + 4 * g + qq];
#pragma unroll
          for (int t = 0; t < TT2; ++t) dst[orow * d.H + 16 * t] = tot[t][qq];
        }
      }
    }
    i = NW + (uint32_t)__builtin_amdgcn_readfirstlane((int)nx);
  }
  stamp_wave(s.tl_experts, kTlPoints, 5 + (wave & 1));
  __syncthreads();
  if (tid == 0) {
    // every block with index x mod kXcds must have run on one XCD: the first
    // of them records its XCC id, the others compare (at the end, so the
    // round trip does not delay the seam; a block on another XCD would have
    // timed out at the barriers)
    const uint32_t id = (__builtin_amdgcn_s_getreg((15 << 11) | 20) & 0xF) + 1u;
    uint32_t prev = 0;
    if (!__hip_atomic_compare_exchange_strong(&s.sync[8 + x], &prev, id, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) &&
        prev != id)
      flag_status(s.status, kStatusXcdMap);
  }
  stamp(s.tl_experts, kTlPoints, 1);
}

// Where the blocks of a launch run: block b stores its XCC id at out[b].
// Launched like the persistent launch (one block of 512 threads per CU).
__global__ __launch_bounds__(512) void xcc_probe_kernel(uint32_t* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = __builtin_amdgcn_s_getreg((15 << 11) | 20) & 0xF;
}


// ROUTE: and the MXFP8 rows of at most kRouteRows tokens
template <bool W13>
size_t gemm_lds(const LayerDims& d, int m, int max_vs, bool route = false) {
  const size_t base = ((size_t)max_vs * 16 + (size_t)(m * d.K + m) * 4 + 15) & ~(size_t)15;
  const size_t mr = m < kRouteRows ? m : kRouteRows;
  if (route) return base + mr * d.H + mr * (d.H / 32);
  return W13 ? base + plan_block_words(d.E) * 4 : base;
}

template <bool W13, int TT, int NW, bool ROUTE = false>
hipError_t launch_gemm_t(const LayerDims& d, int m, const Inputs& in, const Scratch& s, int grid, int max_vs,
                         int split, hipStream_t st, const KernelEvents& ev) {
  return launch_kernel(gemm_kernel<W13, TT, NW, ROUTE>, dim3(grid), dim3(NW * 64),
                       (uint32_t)gemm_lds<W13>(d, m, max_vs, ROUTE), st, ev, d, in, s, m, split, max_vs);
}

template <bool W13, int TT, int NW, bool ROUTE = false>
int occupancy_t(size_t lds) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_kernel<W13, TT, NW, ROUTE>, NW * 64, lds) != hipSuccess)
    return 0;
  return n;
}

}  // namespace

// Nominal waves per block of each GEMM, for the split decision.
int gemm_waves(bool) { return kGemmWaves; }

// The persistent launch's dynamic LDS: slots, row -> token and row -> output
// row, then the MXFP8 rows.
size_t xcd_lds_bytes(const LayerDims& d, int m, int max_vs) {
  const size_t base = ((size_t)max_vs * 16 + (size_t)(m * d.K + m) * 8 + 15) & ~(size_t)15;
  const size_t mr = m < kRouteRows ? m : kRouteRows;
  return base + mr * d.H + mr * (d.H / 32);
}

int xcd_blocks_per_cu(size_t lds) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, xcd_kernel<kGemmWaves>, kGemmWaves * 64, lds) != hipSuccess)
    return 0;
  return n;
}

// Whether the persistent launch covers a step: one that routes inside the
// w13 launch, E4M3 routed experts, and intermediates that cut into kXcds
// slices that are each one w2 segment.
bool xcd_applies(const LayerDims& d, int m, int grid) {
  auto slice_ok = [&d](int Kv) {
    return Kv % (kXcds * 128) == 0 && Kv / (kXcds * 128) == w2_seg_steps(d, Kv, false);
  };
  // a step's slots (the shared one and at most m k routed) number at most
  // 64, the range the launch is measured and tested on
  const bool slots_ok = 1 + std::min(m * d.K, d.E) <= 64;
  return route_in_w13(d, m, grid) && d.rfmt == MOE_DECODE_ROUTED_E4M3 && slice_ok(d.I) && slice_ok(d.Is) &&
         grid % kXcds == 0 && grid / kXcds > 1 && m < kXcds && slots_ok;
}

hipError_t launch_xcd(const LayerDims& d, int m, const Inputs& in, const Scratch& s, int grid, int max_vs,
                      hipStream_t st, const KernelEvents& ev) {
  return launch_kernel(xcd_kernel<kGemmWaves>, dim3(grid), dim3(kGemmWaves * 64),
                       (uint32_t)xcd_lds_bytes(d, m, max_vs), st, ev, d, in, s, m, max_vs);
}

hipError_t probe_xcc(int grid, uint32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(xcc_probe_kernel, dim3(grid), dim3(512), 0, st, out);
  return hipGetLastError();
}

// Tiles per split-mode w2 unit: 8 where a w2 segment is 2 K steps.
int w2_split_tiles(const LayerDims& d) {
  const bool fp4 = d.rfmt == MOE_DECODE_ROUTED_MXFP4;
  return (w2_seg_steps(d, d.I, fp4) == 2 || w2_seg_steps(d, d.Is, false) == 2) ? 8 : kTT2Split;
}

// Split mode when whole units would leave waves without one.  w13: the
// expected slots of a step under uniform routing (E (1 - (1 - K/E)^m)
// distinct experts, plus the shared expert's slots) times the whole units
// of a slot, against 0.9 units per wave (the cases below bracket the cut
// between 0.8 and 1.0).  At H = 5120 on 256 CUs: 64 slots of the
// draft layer (E = 64, k = 4, m = 48) fill 2,048 waves with one unit each
// and run w13 in 112 us whole against 131 us split; a step of 8 rows of the
// 256-expert layer (1.8 units per wave) takes 199 against 206 us; 48 rows at
// I = 256 (0.8 per wave) take 96 whole against 93 us split.  Steps that route
// inside the w13 launch (m <= 4) stay split: there the shared expert's units
// start first, and whole ones (one per wave at m = 4) ended later than the
// split ones (118 against 115 us).  w2: the slot bound min(m k, E) plus the
// shared slots, split under one whole 8-tile unit per wave.
bool gemm_split(const LayerDims& d, int m, int waves, bool w13) {
  const long shared = (m + kTokTile - 1) / kTokTile;
  if (w13) {
    if (m <= kRouteRows) return true;
    const double distinct = d.E * (1.0 - std::pow(1.0 - (double)d.K / d.E, m));
    const double units = (distinct + shared) * (2.0 * d.Imax / 16 / kTT13);
    return units < 0.9 * waves;
  }
  const int pairs = m * d.K;
  const long slots = (long)(pairs < d.E ? pairs : d.E) + shared;
  return slots * (d.H / 16) < 8L * waves;
}

hipError_t launch_w13(const LayerDims& d, int m, const Inputs& in, const Scratch& s, int grid, int max_vs,
                      bool route, hipStream_t st, const KernelEvents& ev) {
  const bool split = gemm_split(d, m, grid * gemm_waves(true), true);
  // the launch that routes: 4 tiles per unit in either mode (registers for
  // its seam)
  if (route) return launch_gemm_t<true, 4, 8, true>(d, m, in, s, grid, max_vs, split ? 1 : 0, st, ev);
  if (split) return launch_gemm_t<true, kTT13, kGemmWaves>(d, m, in, s, grid, max_vs, 1, st, ev);
  return launch_gemm_t<true, kTT13, kGemmWaves>(d, m, in, s, grid, max_vs, 0, st, ev);
}

hipError_t launch_act(const LayerDims& d, int m, const Scratch& s, int w13_grid, hipStream_t st,
                      const KernelEvents& ev) {
  const int split = gemm_split(d, m, w13_grid * gemm_waves(true), true) ? 1 : 0;
  const dim3 grid((d.Imax + kThreads - 1) / kThreads, m * d.K + m), block(kThreads);
  const int nseg = split ? (d.H / 128 + kSegSteps - 1) / kSegSteps : 1;
  if (nseg <= 1) return launch_kernel(act_kernel<1>, grid, block, 0, st, ev, d, s, m, split);
  if (nseg <= 4) return launch_kernel(act_kernel<4>, grid, block, 0, st, ev, d, s, m, split);
  if (nseg <= 12) return launch_kernel(act_kernel<12>, grid, block, 0, st, ev, d, s, m, split);
  return launch_kernel(act_kernel<32>, grid, block, 0, st, ev, d, s, m, split);
}

hipError_t launch_w2(const LayerDims& d, int m, const Inputs& in, const Scratch& s, int grid, int max_vs,
                     hipStream_t st, const KernelEvents& ev) {
  if (gemm_split(d, m, grid * gemm_waves(false), false)) {
    if (w2_split_tiles(d) == 8) return launch_gemm_t<false, 8, kGemmWaves>(d, m, in, s, grid, max_vs, 1, st, ev);
    return launch_gemm_t<false, kTT2Split, kGemmWaves>(d, m, in, s, grid, max_vs, 1, st, ev);
  }
  return launch_gemm_t<false, kTT2Whole, kGemmWaves>(d, m, in, s, grid, max_vs, 0, st, ev);
}

hipError_t launch_combine(const LayerDims& d, int m, const Inputs& in, const Scratch& s, int w2_grid,
                          bool persistent, hipStream_t st, const KernelEvents& ev) {
  // after the persistent launch: its slice planes, and its hand-off words
  // to clear
  const bool clear = persistent;
  const int split = persistent || gemm_split(d, m, w2_grid * gemm_waves(false), false) ? 1 : 0;
  const dim3 grid(d.H / kCombineThreads, m), block(kCombineThreads);
  const int nseg = split ? w2_planes(d) : 1;
  if (nseg <= 1) return launch_kernel(combine_kernel<1>, grid, block, 0, st, ev, d, in, s, m, split, clear ? 1 : 0);
  if (nseg <= 4) return launch_kernel(combine_kernel<4>, grid, block, 0, st, ev, d, in, s, m, split, clear ? 1 : 0);
  if (nseg <= 8) return launch_kernel(combine_kernel<8>, grid, block, 0, st, ev, d, in, s, m, split, clear ? 1 : 0);
  return launch_kernel(combine_kernel<16>, grid, block, 0, st, ev, d, in, s, m, split, clear ? 1 : 0);
}

// Blocks per CU that every variant of the GEMM fits (one block per CU is
// launched; 0 if a variant cannot run with this much LDS).
int gemm_blocks_per_cu(bool w13, size_t lds) {
  int a, b;
  if (w13) {
    a = occupancy_t<true, kTT13, kGemmWaves>(lds);
    b = occupancy_t<true, 4, 8, true>(lds);
  } else {
    a = occupancy_t<false, kTT2Whole, kGemmWaves>(lds);
    b = occupancy_t<false, kTT2Split, kGemmWaves>(lds);
    const int c = occupancy_t<false, 8, kGemmWaves>(lds);
    b = c < b ? c : b;
  }
  return a < b ? a : b;
}

size_t gemm_lds_bytes(const LayerDims& d, int m, int max_vs, bool w13) {
  if (!w13) return gemm_lds<false>(d, m, max_vs);
  const size_t a = gemm_lds<true>(d, m, max_vs, true), b = gemm_lds<true>(d, m, max_vs, false);
  return a > b ? a : b;
}

}  // namespace moe
