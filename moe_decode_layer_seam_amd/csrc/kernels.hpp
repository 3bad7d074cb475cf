// kernels.hpp -- launch interface between the C ABI (api.hip) and the
// kernels (seam.hip, experts.hip, quant.hip).
#pragma once

#include <hip/hip_ext.h>

#include "moe_decode.h"
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Compile-time limits of the kernels (the C ABI validates against them).
constexpr int kMaxTokens = 48;    // DSV41MonoLayer.supports: M <= 48
constexpr int kMaxExperts = 1024;  // 16 sort groups of 64
constexpr int kMaxTopk = 32;       // two top-k lists fit one 64-lane merge
constexpr int kMaxHidden = 16384;
constexpr int kMaxInter = 8192;
constexpr int kTokTile = 16;       // token rows per MFMA tile (one "virtual slot")
constexpr int kThreads = 256;      // blocks of the small kernels

struct LayerDims {
  int H, E, K, I, Is, Imax, Mx;
  float eps, routed_scale;
  int rfmt;  // routed expert weights: MOE_DECODE_ROUTED_E4M3 or _MXFP4
  int xslices;  // plans of the persistent schedule: w2 segments are its XCD slices
};

// The plan's device scratch, laid out for Mx token rows.
struct Scratch {
  uint16_t* normed;   // [Mx, H] bf16
  uint8_t* x8;        // [Mx, H] E4M3
  uint8_t* x8s;       // [Mx, H/32] E8M0
  double* logits;     // [Mx, E]
  int32_t* ids;       // [Mx, K]
  float* wts;         // [Mx, K]
  int32_t* counts;    // [E]
  int32_t* pair_row;  // [Mx, K]
  int32_t* row_tok;   // [R] token of each row; R = Mx*K + Mx
  float* row_w;       // [R] its routing weight (1 for the shared expert)
  int32_t* row_out;   // [R] the row of its w2 sums: pair t k + j, or P + t for the shared row
  int4* vslots;       // [VS] {expert (-1: shared), first row, rows (<= 16), 0}
  int32_t* header;    // [4] {virtual slots, shared virtual slots, routed virtual slots, m}
  uint32_t* counter;  // arrival counter of the route blocks (sync word 0)
  uint8_t* a8;        // [R, Imax] E4M3 SiLU*up intermediate
  uint8_t* a8s;       // [R, Imax/32] E8M0
  float* part13;       // [planes][R][2 Imax] fp32 w13 sums (per K segment in split mode)
  float* part2;        // [planes][R][H] fp32 w2 sums (per K segment in split mode)
  // The hand-off words, nsync from `sync`, zeroed by the seam launch (and
  // after the persistent launch by the combine launch): the route launch's
  // arrival counter (word 0); the persistent launch's XCC ids (words 8..15)
  // and barrier counts (from kXcdBarrierBase, one cache line each); the
  // boxes.
  uint32_t* sync;
  // The run's status word, in its own 256 bytes: bits set by a wait that
  // timed out (kStatus*); sticky across runs until the host clears it.
  uint32_t* status;
  uint32_t* tile_cnt;  // arrivals of the logits launch's blocks per 4-row tile (kTileCntStride apart)
  uint32_t* pick_box;  // [kPickBox] the picks, for the w13 launch that routes (tagged words)
  uint64_t* logit_box; // [kRouteRows][E] its router logits (tagged; E <= 256)
  int nsync;
  // The longest a wait inside a launch spins (100 MHz device-clock ticks)
  // before it sets its status bit and goes on: kWaitTicks, or
  // MOE_DECODE_WAIT_LIMIT_US from the environment.
  uint64_t wait_ticks;
  // timeline records [block][kTlPoints] of each kernel (nullptr: off)
  uint64_t* tl_seam;
  uint64_t* tl_logits;
  uint64_t* tl_route;
  uint64_t* tl_w13;
  uint64_t* tl_act;
  uint64_t* tl_w2;
  uint64_t* tl_combine;
  uint64_t* tl_experts;
};

// Status bits: a wait of the persistent launch for a slot's a8; a wait of
// the w13 launch that routes (or of the persistent launch) for the logits
// or the picks; blocks of the persistent launch with one index mod kXcds
// on different XCDs.
constexpr uint32_t kStatusA8Wait = 1u;
constexpr uint32_t kStatusRouteWait = 2u;
constexpr uint32_t kStatusXcdMap = 4u;
// 100 ms of the 100 MHz device clock: far beyond any real wait.
constexpr uint64_t kWaitTicks = 10000000ull;

constexpr int kKernels = 8;      // seam, logits, route, w13, act, w2, combine, persistent
constexpr int kActCols = 64;     // columns of an act group of the persistent launch
constexpr int kSegSteps = 4;     // K steps of 128 per GEMM segment (w13; w2: w2_seg_steps)

// The persistent launch of small steps cuts the intermediate of every expert
// into kXcds slices, one per XCD.
constexpr int kXcds = 8;
// Its barrier counts: barrier b (0, 1) of XCD x in sync word
// kXcdBarrierBase + (b * kXcds + x) * kXcdBarrierStride, each in a cache line
// of its own.  With the sixteen words in one line, atomics of different
// XCDs on that line held each barrier up for 4-8 us.
constexpr int kXcdBarrierBase = 64;
constexpr int kXcdBarrierStride = 32;  // 128 bytes
constexpr int kXcdBarrierWords = 2 * kXcds * kXcdBarrierStride;
// The logits launch that routes (E <= 64, above four rows): one arrival
// count per 4-row tile, each in a cache line of its own, after the barrier
// words.
constexpr int kTileCntBase = kXcdBarrierBase + kXcdBarrierWords;
constexpr int kTileCntStride = 32;
constexpr int kTileCntWords = (48 + 3) / 4 * kTileCntStride;
// K steps of 128 per segment of a w2 contraction of length Kv (I or Is):
// in plans of the persistent schedule, 2 (256 columns) where Kv is kXcds
// slices of 256, so that those slices are the segments and every step of
// the plan sums w2 in the same order; else kSegSteps (segments of 512
// columns read longer runs of each weight row).  E2M1 weights keep
// kSegSteps: their codes are blocked by 512 columns.
__host__ __device__ inline int w2_seg_steps(const LayerDims& d, int Kv, bool fp4) {
  return (d.xslices && !fp4 && Kv == kXcds * 256) ? 2 : kSegSteps;
}
// Segments of w2 (its sum planes in split mode): the larger of the routed
// and the shared expert's counts.
inline int w2_planes(const LayerDims& d) {
  const int sr = w2_seg_steps(d, d.I, d.rfmt == MOE_DECODE_ROUTED_MXFP4), ss = w2_seg_steps(d, d.Is, false);
  const int nr = (d.I / 128 + sr - 1) / sr, ns = (d.Is / 128 + ss - 1) / ss;
  return nr > ns ? nr : ns;
}

constexpr int kTlPoints = 8;     // stamps per block and kernel
constexpr int kTlBlocks = 1024;  // blocks recorded per kernel (kTlBlockCap)

struct Inputs {
  const uint16_t* x;
  const uint16_t* norm_w;
  const uint16_t* gate_w;
  const float* bias;
  const uint8_t *w13, *w13_s, *w2, *w2_s, *sgu, *sgu_s, *sw2, *sw2_s;
  uint16_t* out;
};

// Upper bound on virtual slots (experts split into tiles of <= 16 rows, the
// shared expert first) for m rows.
inline int max_vslots(int m, int E, int K) {
  int pairs = m * K;
  int routed = (pairs < E ? pairs : E) + (pairs + kTokTile - 1) / kTokTile;
  return routed + (m + kTokTile - 1) / kTokTile;
}

// The seam's thread mapping, shared bit for bit by every kernel that sums a
// row's squares or a router logit (the seam launch, the logits launch and
// the seam inside the w13 launch that routes): 8 columns a thread in chunks
// of kSeamChunk columns, a thread's chunks in order, then the lanes'
// butterfly (32 apart first), then the kSeamWaves waves in order.
constexpr int kSeamThreads = 512;
constexpr int kSeamWaves = kSeamThreads / 64;
constexpr int kSeamChunk = 8 * kSeamThreads;
inline int seam_cpt(int H) { return (H + kSeamChunk - 1) / kSeamChunk; }
// Token rows per block of the seam launch (rows held in registers).
inline int seam_tb(int H) { return seam_cpt(H) <= 2 ? 8 : 4; }
// Experts per block of the seam launch: every block recomputes the norm of
// its rows, so blocks take as many experts as keeps about 256 blocks (and at
// most 256 expert slices).
inline int seam_epb(const LayerDims& d, int m) {
  const long tiles = (m + seam_tb(d.H) - 1) / seam_tb(d.H);
  int epb = d.E <= 256 ? 1 : (d.E <= 512 ? 2 : 4);
  while (epb < 8 && (long)(d.E / (2 * epb)) * tiles >= 256) epb *= 2;
  return epb;
}
// Up to 4 rows the seam launch also computes the router logits (each block
// recomputes the norm of its rows); above, the norm runs once per row and a
// separate launch computes the logits from the stored rows.
inline bool seam_fused(int m) { return m <= 4; }
inline int seam_blocks(const LayerDims& d, int m) {
  const int epb = seam_epb(d, m);
  const int tiles = (m + seam_tb(d.H) - 1) / seam_tb(d.H);
  return seam_fused(m) ? (d.E + epb - 1) / epb * tiles : m;
}
// Steps of at most 4 tokens run the seam and the router inside the w13
// launch instead of launches of their own: every block normalises and
// quantises the rows into its LDS and sums the logits of one or two experts,
// the first m blocks route (one per token), and the others start on the
// shared expert.  When the router's expert groups fit its four waves, the
// plan fits one wave (at most 64 pairs), a row fits two chunks of the seam's
// thread mapping, and two experts per block cover E.
constexpr int kRouteRows = 4;
inline bool route_in_w13(const LayerDims& d, int m, int grid) {
  return m <= kRouteRows && m * d.K <= 64 && d.E <= 256 && d.H <= 8192 && d.E <= 2 * grid && grid > m;
}
// The picks as the w13 launch that routes reads them: word t k + j holds the
// expert of token t's pick j with bit 31 set.  The box is zeroed before each
// step, so a reader knows a word is in from the word alone.
constexpr int kPickBox = 64;
constexpr uint32_t kBoxTag = 0x80000000u;
// A logit in the logit box: its bits with the sign bit flipped.  A logit is
// a sum that starts from +0, so it is never -0 and its word never 0 (the
// zeroed box's value).
constexpr uint64_t kLogitTag = 0x8000000000000000ull;
inline int logits_blocks(const LayerDims& d, int m) {
  const int tb = 4, epb = seam_cpt(d.H) <= 2 ? 4 : 2;
  return seam_fused(m) ? 0 : (d.E + epb - 1) / epb * ((m + tb - 1) / tb);
}

// Optional timing events of one launch: when `start` is set the dispatch
// itself records them (hipExtLaunchKernelGGL), so their interval is the
// kernel's execution, without the queue latency of separate event packets.
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

template <typename F, typename... A>
inline hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st,
                                const KernelEvents& ev, A... args) {
  if (ev.start)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
  return hipGetLastError();
}

// Launchers; each returns the hipError_t of its launch.
hipError_t launch_seam(const LayerDims& d, int m, const Inputs& in, const Scratch& s, hipStream_t st,
                       const KernelEvents& ev);
hipError_t launch_logits(const LayerDims& d, int m, const Inputs& in, const Scratch& s, bool route, hipStream_t st,
                         const KernelEvents& ev);
// plan: the route launch also builds the plan (last block to finish); else
// the w13 launch builds it from the stored picks.
hipError_t launch_route(const LayerDims& d, int m, const Inputs& in, const Scratch& s, bool plan, hipStream_t st,
                        const KernelEvents& ev);
// route: the launch also runs the seam and routes (route_in_w13): its first
// m blocks run the router while the others stream the shared expert's units.
hipError_t launch_w13(const LayerDims& d, int m, const Inputs& in, const Scratch& s, int grid, int max_vs,
                      bool route, hipStream_t st, const KernelEvents& ev);
hipError_t launch_act(const LayerDims& d, int m, const Scratch& s, int w13_grid, hipStream_t st,
                      const KernelEvents& ev);
hipError_t launch_w2(const LayerDims& d, int m, const Inputs& in, const Scratch& s, int grid, int max_vs,
                     hipStream_t st, const KernelEvents& ev);
// persistent: after the persistent launch (its w2 slice planes; also clear
// its hand-off words for the next step)
hipError_t launch_combine(const LayerDims& d, int m, const Inputs& in, const Scratch& s, int w2_grid,
                          bool persistent, hipStream_t st, const KernelEvents& ev);
// The persistent launch of a step of at most kRouteRows rows (seam, router,
// w13, SiLU * up and w2), cut by XCD: whether it covers a step, its launch,
// its dynamic LDS and occupancy.  probe_xcc: block b of a grid of `grid`
// blocks of 512 threads stores its XCC id at out[b] (the plan checks that
// blocks are dealt to the XCDs round-robin).
bool xcd_applies(const LayerDims& d, int m, int grid);
hipError_t launch_xcd(const LayerDims& d, int m, const Inputs& in, const Scratch& s, int grid, int max_vs,
                      hipStream_t st, const KernelEvents& ev);
size_t xcd_lds_bytes(const LayerDims& d, int m, int max_vs);
int xcd_blocks_per_cu(size_t lds);
hipError_t probe_xcc(int grid, uint32_t* out, hipStream_t st);
// Whether a step of m rows runs the GEMM (w13 or w2) in split mode on
// `waves` waves, the occupancy of its kernel and its dynamic LDS bytes.
bool gemm_split(const LayerDims& d, int m, int waves, bool w13);
int gemm_blocks_per_cu(bool w13, size_t lds);
int gemm_waves(bool w13);  // waves per block of the GEMM
size_t gemm_lds_bytes(const LayerDims& d, int m, int max_vs, bool w13);
hipError_t launch_quant_weight(const float* w, int count, int rows, int cols, uint8_t* q, uint8_t* sc,
                               hipStream_t st);
// The seam upstream of the MoE (hc.hip): the hyper-connection residual fold
// and the attention seam's MXFP8.
hipError_t launch_hc_fold(int m, int H, const uint16_t* part, const uint16_t* residual, const float* post,
                          const float* res, const float* pre, uint16_t* residual_out, uint16_t* x, hipStream_t st);
hipError_t launch_attn_x8(int m, int H, const uint16_t* x, const uint16_t* w, float eps, uint8_t* x8, uint8_t* x8s,
                          hipStream_t st);
// MXFP4 of count [rows, cols] matrices (rows % 16 == 0, cols % 32 == 0):
// E2M1 pairs and blocked codes [rows/16][ceil(cols/512)][16][16] each.
hipError_t launch_quant_weight_fp4(const float* w, int count, int rows, int cols, uint8_t* q, uint8_t* sc,
                                   hipStream_t st);

}  // namespace moe
