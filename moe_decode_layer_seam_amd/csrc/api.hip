// api.hip -- the C ABI (include/moe_decode.h): plan (validation, scratch
// layout, one allocation), run (argument checks, three launches on the
// caller's stream, no allocation, no synchronisation), inspect, timing.
//
// Pages: "vllm.models.deepseek_v41.amd.mono.runner" DSV41MonoLayer.ffn (one
// launch set per step on the caller's stream; every argument a device
// pointer, so the launches can be captured in a HIP graph),
// DSV41MonoLayer.scratch (scratch sized for a step width and allocated
// before any capture), DSV41MonoLayer.supports (1 <= M <= 48),
// _check_tensors (argument checks, since the kernels' loads are unchecked).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "moe_decode.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
constexpr int kTimingRing = 256;  // runs whose events are held before folding

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct TimingSet {
  hipEvent_t ev[2 * kKernels];  // start and stop of each kernel's dispatch
  uint32_t launched = 0;        // kernels of the run (bit k), whose events were recorded
};

std::string g_last_error = "no error";

}  // namespace

struct moe_decode_plan_s {
  LayerDims d{};
  int device = 0;
  int cus = 0;
  int grid13 = 0, grid2 = 0;  // blocks of the w13 and w2 launches
  int max_vs = 0;
  int R = 0;
  size_t bytes = 0;
  void* base = nullptr;
  Scratch s{};
  int last_m = 0;
  int last_grid[kKernels] = {};
  bool boxes_dirty = false;  // a launch that routes ran without the launch after it that clears its boxes
  bool persistent = false;   // the persistent launch serves the steps it covers (checked dispatch)
  bool timeline = false;
  uint64_t* tl_base = nullptr;  // [kKernels][kTlBlocks][kTlPoints]
  std::string err = "no error";
  // timing
  bool timing = false;
  std::vector<TimingSet> ring;
  int ring_used = 0;
  double total_ms[kKernels] = {};
  int runs[kKernels] = {};
};

namespace {

int hip_fail(moe_decode_plan_s* p, hipError_t e, const char* what) {
  std::string msg = std::string(what) + ": " + hipGetErrorString(e);
  if (p) p->err = msg;
  g_last_error = msg;
  return MOE_DECODE_EHIP;
}

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dims(const moe_decode_dims* d) {
  if (!d) return false;
  if (d->hidden < 128 || d->hidden > kMaxHidden || d->hidden % 128) return false;
  if (d->experts < 1 || d->experts > kMaxExperts) return false;
  if (d->topk < 1 || d->topk > kMaxTopk || d->topk > d->experts) return false;
  if (d->inter < 128 || d->inter > kMaxInter || d->inter % 128) return false;
  if (d->shared_inter < 128 || d->shared_inter > kMaxInter || d->shared_inter % 128) return false;
  if (d->max_tokens < 1 || d->max_tokens > kMaxTokens) return false;
  if (!std::isfinite(d->rms_eps) || d->rms_eps < 0.0f) return false;
  if (!std::isfinite(d->routed_scale)) return false;
  if (d->routed_format != MOE_DECODE_ROUTED_E4M3 && d->routed_format != MOE_DECODE_ROUTED_MXFP4) return false;
  if (d->schedule != MOE_DECODE_SCHEDULE_AUTO && d->schedule != MOE_DECODE_SCHEDULE_LAUNCHES &&
      d->schedule != MOE_DECODE_SCHEDULE_PERSISTENT)
    return false;
  return true;
}

// Fold finished timing events into the totals (oldest first).
void fold_timing(moe_decode_plan_s* p) {
  for (int i = 0; i < p->ring_used; ++i) {
    TimingSet& t = p->ring[i];
    for (int k = 0; k < kKernels; ++k)
      if ((t.launched >> k) & 1u) (void)hipEventSynchronize(t.ev[2 * k + 1]);
    for (int k = 0; k < kKernels; ++k) {
      float ms = 0.0f;
      if (((t.launched >> k) & 1u) && hipEventElapsedTime(&ms, t.ev[2 * k], t.ev[2 * k + 1]) == hipSuccess) {
        p->total_ms[k] += ms;
        p->runs[k] += 1;
      }
    }
    t.launched = 0;
  }
  p->ring_used = 0;
}

void free_timing(moe_decode_plan_s* p) {
  for (auto& t : p->ring)
    for (auto& e : t.ev) (void)hipEventDestroy(e);
  p->ring.clear();
  p->ring_used = 0;
}

}  // namespace

namespace moe {
// probe.hip: the streaming read of `bytes` (a multiple of 16) from buf by
// MOE_DECODE_PROBE_BLOCKS blocks, each storing the XOR of the words it read
// at sink[block].
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);
}  // namespace moe

namespace {

// Byte offsets of the scratch regions of one layout, each 256-byte aligned.
struct Layout {
  size_t normed, x8, x8s, logits, ids, wts, counts, pair, tok, roww, rowout, vs, hdr, a8, a8s;
  size_t sync, status, tl, part13, part2, bytes;
  size_t nsync, lbox;  // words of the hand-off region; the logit box's first word
};

// The layout for d.Mx token rows: GEMM sum planes sized for every step
// width up to d.Mx (one [R(m)][width] fp32 plane, or one per K segment for
// the widths that run in split mode or in the persistent launch, where
// `persistent` says it may serve them); `timeline`: room for the stamps.
Layout make_layout(const LayerDims& d, int max_vs, int grid13, int grid2, bool timeline, bool persistent) {
  Layout L{};
  const size_t Mx = d.Mx, H = d.H, E = d.E, K = d.K, R = Mx * K + Mx;
  size_t off = 0;
  auto take = [&](size_t n) {
    size_t o = off;
    off = align_up(off + n);
    return o;
  };
  L.normed = take(Mx * H * 2), L.x8 = take(Mx * H), L.x8s = take(Mx * H / 32);
  L.logits = take(Mx * E * 8), L.ids = take(Mx * K * 4), L.wts = take(Mx * K * 4);
  L.counts = take(E * 4), L.pair = take(Mx * K * 4), L.tok = take(R * 4), L.roww = take(R * 4);
  L.rowout = take(R * 4);
  L.vs = take((size_t)max_vs * 16), L.hdr = take(16);
  L.a8 = take(R * d.Imax), L.a8s = take(R * d.Imax / 32);
  // the hand-off words, zeroed by the seam launch: the route launch's arrival
  // counter (word 0), the XCC id + 1 seen by the persistent launch's blocks
  // of each index mod kXcds (words 8..15), from word 64 that launch's two
  // barrier counts per XCD (a cache line each), then the boxes of the
  // launches that route: the pick box, then (from an even word) the logit box
  L.lbox = (kTileCntBase + kTileCntWords + (size_t)kPickBox + 1) & ~(size_t)1;
  L.nsync = L.lbox + (d.E <= 256 ? (size_t)2 * kRouteRows * d.E : 0);
  L.sync = take(L.nsync * 4);
  L.status = take(4);
  L.tl = timeline ? take((size_t)kKernels * kTlBlocks * kTlPoints * 8) : 0;
  size_t part13 = 0, part2 = 0;
  const size_t nseg13 = (H / 128 + kSegSteps - 1) / kSegSteps;
  const size_t nseg2 = (size_t)w2_planes(d);
  for (int mm = 1; mm <= d.Mx; ++mm) {
    const size_t Rm = (size_t)mm * (K + 1);
    const bool xcd = persistent && xcd_applies(d, mm, grid13);
    const size_t a = (xcd || gemm_split(d, mm, grid13 * gemm_waves(true), true) ? nseg13 : 1) * Rm * 2 * d.Imax * 4;
    const size_t c = (xcd || gemm_split(d, mm, grid2 * gemm_waves(false), false) ? nseg2 : 1) * Rm * H * 4;
    part13 = a > part13 ? a : part13;
    part2 = c > part2 ? c : part2;
  }
  L.part13 = take(part13), L.part2 = take(part2);
  L.bytes = off;
  return L;
}

// The kernels' view of a layout at device address b.
// The bound of the waits inside a launch: MOE_DECODE_WAIT_LIMIT_US (whole
// microseconds) when set, else kWaitTicks.  A small bound makes the waits
// give up at once (their status bits report it): a way to check that path.
uint64_t wait_ticks_from_env() {
  const char* v = std::getenv("MOE_DECODE_WAIT_LIMIT_US");
  if (!v || !*v) return kWaitTicks;
  char* end = nullptr;
  const unsigned long long us = std::strtoull(v, &end, 10);
  if (!end || *end || us > kWaitTicks / 100) return kWaitTicks;
  return (uint64_t)us * 100;
}

Scratch scratch_at(char* b, const Layout& L, const LayerDims& d, int max_vs) {
  Scratch s{};
  s.wait_ticks = wait_ticks_from_env();
  s.normed = reinterpret_cast<uint16_t*>(b + L.normed);
  s.x8 = reinterpret_cast<uint8_t*>(b + L.x8);
  s.x8s = reinterpret_cast<uint8_t*>(b + L.x8s);
  s.logits = reinterpret_cast<double*>(b + L.logits);
  s.ids = reinterpret_cast<int32_t*>(b + L.ids);
  s.wts = reinterpret_cast<float*>(b + L.wts);
  s.counts = reinterpret_cast<int32_t*>(b + L.counts);
  s.pair_row = reinterpret_cast<int32_t*>(b + L.pair);
  s.row_tok = reinterpret_cast<int32_t*>(b + L.tok);
  s.row_w = reinterpret_cast<float*>(b + L.roww);
  s.row_out = reinterpret_cast<int32_t*>(b + L.rowout);
  s.vslots = reinterpret_cast<int4*>(b + L.vs);
  s.header = reinterpret_cast<int32_t*>(b + L.hdr);
  s.a8 = reinterpret_cast<uint8_t*>(b + L.a8);
  s.a8s = reinterpret_cast<uint8_t*>(b + L.a8s);
  s.part13 = reinterpret_cast<float*>(b + L.part13);
  s.part2 = reinterpret_cast<float*>(b + L.part2);
  s.sync = reinterpret_cast<uint32_t*>(b + L.sync);
  s.counter = s.sync;
  s.status = reinterpret_cast<uint32_t*>(b + L.status);
  s.tile_cnt = s.sync + kTileCntBase;
  s.pick_box = s.sync + kTileCntBase + kTileCntWords;
  s.logit_box = d.E <= 256 ? reinterpret_cast<uint64_t*>(s.sync + L.lbox) : nullptr;
  s.nsync = (int)L.nsync;
  return s;
}

LayerDims dims_of(const moe_decode_dims* dims) {
  LayerDims d{};
  d.H = dims->hidden;
  d.E = dims->experts;
  d.K = dims->topk;
  d.I = dims->inter;
  d.Is = dims->shared_inter;
  d.Imax = d.I > d.Is ? d.I : d.Is;
  d.Mx = dims->max_tokens;
  d.eps = dims->rms_eps;
  d.routed_scale = dims->routed_scale;
  d.rfmt = dims->routed_format;
  d.xslices = dims->schedule == MOE_DECODE_SCHEDULE_PERSISTENT ? 1 : 0;
  return d;
}

// Whether every GEMM variant fits a CU once (the expert GEMMs run one block
// per CU).
bool fits_cu(const LayerDims& d, int max_vs) {
  return gemm_blocks_per_cu(true, gemm_lds_bytes(d, d.Mx, max_vs, true)) >= 1 &&
         gemm_blocks_per_cu(false, gemm_lds_bytes(d, d.Mx, max_vs, false)) >= 1;
}

// The argument checks of a run (nothing is enqueued when one fails).
const char* check_run(const LayerDims& d, int m, int max_m, const void* const* ptrs, int nptrs, const void* d_x,
                      const void* d_out) {
  if (m < 1 || m > max_m) return "m outside [1, max_tokens]";
  for (int i = 0; i < nptrs; ++i)
    if (!aligned16(ptrs[i])) return "null or misaligned (not 16-byte) pointer";
  // out is written while x is still read by other blocks: no overlap
  const uintptr_t xo = reinterpret_cast<uintptr_t>(d_x), oo = reinterpret_cast<uintptr_t>(d_out);
  const uintptr_t n = (uintptr_t)m * d.H * 2;
  if (xo < oo + n && oo < xo + n) return "out overlaps x";
  return nullptr;
}

Inputs inputs_of(const void* d_x, const void* d_norm_w, const void* d_gate_w, const float* d_bias, const void* d_w13,
                 const void* d_w13_s, const void* d_w2, const void* d_w2_s, const void* d_sgu, const void* d_sgu_s,
                 const void* d_sw2, const void* d_sw2_s, void* d_out) {
  Inputs in;
  in.x = static_cast<const uint16_t*>(d_x);
  in.norm_w = static_cast<const uint16_t*>(d_norm_w);
  in.gate_w = static_cast<const uint16_t*>(d_gate_w);
  in.bias = d_bias;
  in.w13 = static_cast<const uint8_t*>(d_w13);
  in.w13_s = static_cast<const uint8_t*>(d_w13_s);
  in.w2 = static_cast<const uint8_t*>(d_w2);
  in.w2_s = static_cast<const uint8_t*>(d_w2_s);
  in.sgu = static_cast<const uint8_t*>(d_sgu);
  in.sgu_s = static_cast<const uint8_t*>(d_sgu_s);
  in.sw2 = static_cast<const uint8_t*>(d_sw2);
  in.sw2_s = static_cast<const uint8_t*>(d_sw2_s);
  in.out = static_cast<uint16_t*>(d_out);
  return in;
}

// One step's launches on st.  persistent: the persistent launch may serve
// the step (if it covers it).  seam_always: launch the seam even where a
// later launch runs it itself (the seam launch zeroes the hand-off words).
// boxes_dirty (may be null): set while a launch that routes has run
// without the launch after it that clears its boxes.  ts (may be null): the
// run's timing events; last_grid (may be null): the launches' grids.
hipError_t enqueue(const LayerDims& d, int m, const Inputs& in, const Scratch& sc, int grid13, int grid2, int max_vs,
                   bool persistent, bool seam_always, bool* boxes_dirty, TimingSet* ts, int* last_grid,
                   hipStream_t st, const char** what) {
  const bool fused = persistent && xcd_applies(d, m, grid13);
  const bool route13 = fused || route_in_w13(d, m, grid13);
  const bool seam = !route13 || seam_always || (boxes_dirty && *boxes_dirty);
  if (last_grid) {
    last_grid[0] = seam ? seam_blocks(d, m) : 0;
    last_grid[1] = logits_blocks(d, m);
    last_grid[2] = m;
    last_grid[3] = grid13;
    last_grid[4] = (d.Imax + kThreads - 1) / kThreads * (m * d.K + m);
    last_grid[5] = grid2;
    last_grid[6] = d.H / 64 * m;
    last_grid[7] = grid13;
  }
  auto ev = [&](int k) {
    KernelEvents r;
    if (ts) {
      r.start = ts->ev[2 * k], r.stop = ts->ev[2 * k + 1];
      ts->launched |= 1u << k;
    }
    return r;
  };
  hipError_t e;
  if (seam && (e = launch_seam(d, m, in, sc, st, ev(0))) != hipSuccess) return *what = "seam launch", e;
  // with one sort group (E <= 64) the logits launch routes each 4-row tile
  // in its last block, and no route launch runs
  const bool route_logits = !route13 && !seam_fused(m) && d.E <= 64;
  if (!seam_fused(m) && (e = launch_logits(d, m, in, sc, route_logits, st, ev(1))) != hipSuccess)
    return *what = "logits launch", e;
  // the launches that route build their own plan from the stored picks
  if (!route13 && !route_logits && (e = launch_route(d, m, in, sc, false, st, ev(2))) != hipSuccess)
    return *what = "route launch", e;
  if (route13 && boxes_dirty) *boxes_dirty = true;
  if (fused) {
    if ((e = launch_xcd(d, m, in, sc, grid13, max_vs, st, ev(7))) != hipSuccess)
      return *what = "persistent launch", e;
  } else {
    if ((e = launch_w13(d, m, in, sc, grid13, max_vs, route13, st, ev(3))) != hipSuccess)
      return *what = "w13 launch", e;
    if ((e = launch_act(d, m, sc, grid13, st, ev(4))) != hipSuccess) return *what = "act launch", e;
    if (boxes_dirty) *boxes_dirty = false;
    if ((e = launch_w2(d, m, in, sc, grid2, max_vs, st, ev(5))) != hipSuccess) return *what = "w2 launch", e;
  }
  if ((e = launch_combine(d, m, in, sc, grid2, fused, st, ev(6))) != hipSuccess) return *what = "combine launch", e;
  if (fused && boxes_dirty) *boxes_dirty = false;
  return hipSuccess;
}

// The scratch of moe_decode_run_noalloc: one array per GPU the library runs
// on, held until the process ends.  Its name is a host-side stand-in; host
// code uses the device address hipGetSymbolAddress gives, kept per device.
constexpr size_t kNoAllocBytes = MOE_DECODE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
struct NoAllocDevice {
  char* ptr = nullptr;  // the array's device address on this device
  int cus = 0;
};
NoAllocDevice g_noalloc[kMaxDevices];
std::mutex g_noalloc_mu;

}  // namespace

extern "C" {

int moe_decode_plan(const moe_decode_dims* dims, void* stream, moe_decode_handle* out) {
  if (!out) return MOE_DECODE_EINVAL;
  *out = nullptr;
  if (!valid_dims(dims)) {
    g_last_error = "invalid dimensions";
    return MOE_DECODE_EINVAL;
  }
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cap);
  if (e != hipSuccess) return hip_fail(nullptr, e, "hipStreamIsCapturing");
  if (cap != hipStreamCaptureStatusNone) {
    g_last_error = "moe_decode_plan called during stream capture";
    return MOE_DECODE_ECAPTURE;
  }
  auto* p = new (std::nothrow) moe_decode_plan_s();
  if (!p) return MOE_DECODE_ENOMEM;
  LayerDims& d = p->d;
  d = dims_of(dims);
  p->max_vs = max_vslots(d.Mx, d.E, d.K);
  p->R = d.Mx * d.K + d.Mx;

  if ((e = hipGetDevice(&p->device)) != hipSuccess) {
    int rc = hip_fail(p, e, "hipGetDevice");
    delete p;
    return rc;
  }
  if ((e = hipDeviceGetAttribute(&p->cus, hipDeviceAttributeMultiprocessorCount, p->device)) != hipSuccess) {
    int rc = hip_fail(p, e, "hipDeviceGetAttribute");
    delete p;
    return rc;
  }
  if (!fits_cu(d, p->max_vs)) {
    p->err = g_last_error = "the expert GEMM blocks do not fit a CU for these dimensions";
    delete p;
    return MOE_DECODE_EINVAL;
  }
  p->grid13 = p->grid2 = p->cus;
  const Layout L = make_layout(d, p->max_vs, p->grid13, p->grid2, true,
                               dims->schedule == MOE_DECODE_SCHEDULE_PERSISTENT);
  p->bytes = L.bytes;
  if ((e = hipMalloc(&p->base, p->bytes)) != hipSuccess) {
    hip_fail(p, e, "hipMalloc");
    delete p;
    return MOE_DECODE_ENOMEM;
  }
  if ((e = hipMemset(p->base, 0, p->bytes)) != hipSuccess) {
    int rc = hip_fail(p, e, "hipMemset");
    (void)hipFree(p->base);
    delete p;
    return rc;
  }
  char* b = static_cast<char*>(p->base);
  p->s = scratch_at(b, L, d, p->max_vs);
  p->tl_base = reinterpret_cast<uint64_t*>(b + L.tl);
  // the persistent launch serves the steps it covers if its blocks fit a CU
  // and the device deals a launch's blocks to the XCDs round-robin, from
  // whichever XCD the previous launch left off at (checked here with a probe
  // launch that stores each block's XCC id into the scratch, then zeroed
  // again): then the blocks with one index mod kXcds share an XCD
  if (dims->schedule == MOE_DECODE_SCHEDULE_PERSISTENT && p->grid13 % kXcds == 0 && p->grid13 <= 4096 &&
      xcd_blocks_per_cu(xcd_lds_bytes(d, d.Mx < kRouteRows ? d.Mx : kRouteRows, p->max_vs)) >= 1 &&
      p->bytes >= (size_t)p->grid13 * 4) {
    std::vector<uint32_t> ids((size_t)p->grid13);
    uint32_t* dev_ids = reinterpret_cast<uint32_t*>(b);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((e = probe_xcc(p->grid13, dev_ids, st)) != hipSuccess ||
        (e = hipMemcpyAsync(ids.data(), dev_ids, ids.size() * 4, hipMemcpyDeviceToHost, st)) != hipSuccess ||
        (e = hipStreamSynchronize(st)) != hipSuccess ||
        (e = hipMemsetAsync(dev_ids, 0, ids.size() * 4, st)) != hipSuccess ||
        (e = hipStreamSynchronize(st)) != hipSuccess) {
      int rc = hip_fail(p, e, "dispatch probe");
      (void)hipFree(p->base);
      delete p;
      return rc;
    }
    bool rr = true;
    for (size_t i = 0; i < ids.size(); ++i) rr = rr && ids[i] == (ids[0] + (uint32_t)i) % kXcds;
    p->persistent = rr;
  }
  *out = p;
  return MOE_DECODE_OK;
}

size_t moe_decode_scratch_bytes(moe_decode_handle p) { return p ? p->bytes : 0; }

int moe_decode_run(moe_decode_handle p, int32_t m, const void* d_x, const void* d_norm_w, const void* d_gate_w,
                   const float* d_bias, const void* d_w13, const void* d_w13_s, const void* d_w2,
                   const void* d_w2_s, const void* d_sgu, const void* d_sgu_s, const void* d_sw2,
                   const void* d_sw2_s, void* d_out, void* stream) {
  if (!p) return MOE_DECODE_EINVAL;
  const LayerDims& d = p->d;
  const void* ptrs[] = {d_x, d_norm_w, d_gate_w, d_bias, d_w13, d_w13_s, d_w2, d_w2_s,
                        d_sgu, d_sgu_s, d_sw2, d_sw2_s, d_out};
  if (const char* why = check_run(d, m, d.Mx, ptrs, 13, d_x, d_out)) {
    p->err = why;
    return MOE_DECODE_EINVAL;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Inputs in = inputs_of(d_x, d_norm_w, d_gate_w, d_bias, d_w13, d_w13_s, d_w2, d_w2_s, d_sgu, d_sgu_s, d_sw2,
                              d_sw2_s, d_out);
  TimingSet* ts = nullptr;
  if (p->timing) {
    if (p->ring_used == kTimingRing) fold_timing(p);
    ts = &p->ring[p->ring_used++];
  }
  Scratch sc = p->s;
  if (p->timeline) {
    uint64_t* tl[kKernels];
    for (int k = 0; k < kKernels; ++k) tl[k] = p->tl_base + (size_t)k * kTlBlocks * kTlPoints;
    sc.tl_seam = tl[0];
    sc.tl_logits = tl[1];
    sc.tl_route = tl[2];
    sc.tl_w13 = tl[3];
    sc.tl_act = tl[4];
    sc.tl_w2 = tl[5];
    sc.tl_combine = tl[6];
    sc.tl_experts = tl[7];
  }
  const char* what = "";
  hipError_t e = enqueue(d, m, in, sc, p->grid13, p->grid2, p->max_vs, p->persistent, false, &p->boxes_dirty, ts,
                         p->last_grid, st, &what);
  if (e != hipSuccess) return hip_fail(p, e, what);
  p->last_m = m;
  return MOE_DECODE_OK;
}

int moe_decode_run_noalloc(const moe_decode_dims* dims, int32_t m, const void* d_x, const void* d_norm_w,
                           const void* d_gate_w, const float* d_bias, const void* d_w13, const void* d_w13_s,
                           const void* d_w2, const void* d_w2_s, const void* d_sgu, const void* d_sgu_s,
                           const void* d_sw2, const void* d_sw2_s, void* d_out, uint32_t* d_status, void* stream) {
  if (!valid_dims(dims)) {
    g_last_error = "invalid dimensions";
    return MOE_DECODE_EINVAL;
  }
  LayerDims d = dims_of(dims);
  const void* ptrs[] = {d_x, d_norm_w, d_gate_w, d_bias, d_w13, d_w13_s, d_w2, d_w2_s,
                        d_sgu, d_sgu_s, d_sw2, d_sw2_s, d_out};
  if (const char* why = check_run(d, m, d.Mx, ptrs, 13, d_x, d_out)) {
    g_last_error = why;
    return MOE_DECODE_EINVAL;
  }
  if (d_status == nullptr || reinterpret_cast<uintptr_t>(d_status) % 4) {
    g_last_error = "null or misaligned status word";
    return MOE_DECODE_EINVAL;
  }
  // this step's layout only: its rows, not max_tokens'
  d.Mx = m;
  const int max_vs = max_vslots(d.Mx, d.E, d.K);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(nullptr, e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    g_last_error = "device index beyond the no-alloc table";
    return MOE_DECODE_EINVAL;
  }
  NoAllocDevice nd;
  {
    // once per device, with it current: the array's address on this device
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    if (g_noalloc[dev].ptr == nullptr) {
      void* ptr = nullptr;
      if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess)
        return hip_fail(nullptr, e, "hipGetSymbolAddress");
      int cus = 0;
      if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
        return hip_fail(nullptr, e, "hipDeviceGetAttribute");
      g_noalloc[dev].ptr = static_cast<char*>(ptr);
      g_noalloc[dev].cus = cus;
    }
    nd = g_noalloc[dev];
  }
  if (!fits_cu(d, max_vs)) {
    g_last_error = "the expert GEMM blocks do not fit a CU for these dimensions";
    return MOE_DECODE_EINVAL;
  }
  const Layout L = make_layout(d, max_vs, nd.cus, nd.cus, false, false);
  if (L.bytes > kNoAllocBytes) {
    g_last_error = "the step's scratch exceeds MOE_DECODE_NOALLOC_SCRATCH_BYTES";
    return MOE_DECODE_EINVAL;
  }
  Scratch sc = scratch_at(nd.ptr, L, d, max_vs);
  sc.status = d_status;
  const Inputs in = inputs_of(d_x, d_norm_w, d_gate_w, d_bias, d_w13, d_w13_s, d_w2, d_w2_s, d_sgu, d_sgu_s, d_sw2,
                              d_sw2_s, d_out);
  // the seam launch runs in every step: it zeroes the hand-off words, which
  // the array holds from whatever call used it last.  The short launches
  // serve every step here: the persistent launch needs the dispatch check a
  // plan makes (which synchronises, and may not run under capture); a
  // token's output bits are the same either way.
  const char* what = "";
  e = enqueue(d, m, in, sc, nd.cus, nd.cus, max_vs, false, true, nullptr, nullptr, nullptr,
              static_cast<hipStream_t>(stream), &what);
  if (e != hipSuccess) return hip_fail(nullptr, e, what);
  return MOE_DECODE_OK;
}

int moe_decode_status(moe_decode_handle p, void* stream, uint32_t* h_status, int32_t clear) {
  if (!p || !h_status) return MOE_DECODE_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(st, &cap);
  if (e != hipSuccess) return hip_fail(p, e, "hipStreamIsCapturing");
  if (cap != hipStreamCaptureStatusNone) {
    p->err = "moe_decode_status called during stream capture";
    return MOE_DECODE_ECAPTURE;
  }
  uint32_t v = 0;
  if ((e = hipMemcpyAsync(&v, p->s.status, 4, hipMemcpyDeviceToHost, st)) != hipSuccess ||
      (e = hipStreamSynchronize(st)) != hipSuccess)
    return hip_fail(p, e, "status read");
  if (clear && v != 0u) {
    if ((e = hipMemsetAsync(p->s.status, 0, 4, st)) != hipSuccess || (e = hipStreamSynchronize(st)) != hipSuccess)
      return hip_fail(p, e, "status clear");
  }
  *h_status = v;
  return MOE_DECODE_OK;
}

int moe_decode_inspect(moe_decode_handle p, int32_t tap, const void** d_ptr, size_t* bytes) {
  if (!p || !d_ptr || !bytes) return MOE_DECODE_EINVAL;
  const LayerDims& d = p->d;
  const size_t m = p->last_m > 0 ? p->last_m : d.Mx;
  const size_t H = d.H, E = d.E, K = d.K, R = m * K + m;
  const Scratch& s = p->s;
  switch (tap) {
    case MOE_DECODE_TAP_NORMED: *d_ptr = s.normed; *bytes = m * H * 2; break;
    case MOE_DECODE_TAP_X8: *d_ptr = s.x8; *bytes = m * H; break;
    case MOE_DECODE_TAP_X8S: *d_ptr = s.x8s; *bytes = m * H / 32; break;
    case MOE_DECODE_TAP_LOGITS: *d_ptr = s.logits; *bytes = m * E * 8; break;
    case MOE_DECODE_TAP_TOPK_IDS: *d_ptr = s.ids; *bytes = m * K * 4; break;
    case MOE_DECODE_TAP_TOPK_W: *d_ptr = s.wts; *bytes = m * K * 4; break;
    case MOE_DECODE_TAP_COUNTS: *d_ptr = s.counts; *bytes = E * 4; break;
    case MOE_DECODE_TAP_PAIR_ROW: *d_ptr = s.pair_row; *bytes = m * K * 4; break;
    case MOE_DECODE_TAP_ROW_TOK: *d_ptr = s.row_tok; *bytes = R * 4; break;
    case MOE_DECODE_TAP_A8: *d_ptr = s.a8; *bytes = R * d.Imax; break;
    case MOE_DECODE_TAP_A8S: *d_ptr = s.a8s; *bytes = R * d.Imax / 32; break;
    case MOE_DECODE_TAP_STATUS: *d_ptr = s.status; *bytes = 4; break;
    default: return MOE_DECODE_EINVAL;
  }
  return MOE_DECODE_OK;
}

int moe_decode_timing(moe_decode_handle p, int32_t on) {
  if (!p) return MOE_DECODE_EINVAL;
  if (on) {
    if (p->ring.empty()) {
      p->ring.resize(kTimingRing);
      for (auto& t : p->ring)
        for (auto& ev : t.ev) {
          hipError_t e = hipEventCreate(&ev);
          if (e != hipSuccess) {
            free_timing(p);
            return hip_fail(p, e, "hipEventCreate");
          }
        }
    }
    fold_timing(p);
    for (double& t : p->total_ms) t = 0.0;
    for (int& r : p->runs) r = 0;
    p->timing = true;
  } else {
    p->timing = false;
  }
  return MOE_DECODE_OK;
}

int moe_decode_timing_read(moe_decode_handle p, int32_t kernel, double* total_ms, int32_t* runs) {
  if (!p || kernel < 0 || kernel >= kKernels || !total_ms || !runs) return MOE_DECODE_EINVAL;
  fold_timing(p);
  *total_ms = p->total_ms[kernel];
  *runs = p->runs[kernel];
  return MOE_DECODE_OK;
}

int moe_decode_timeline(moe_decode_handle p, int32_t on) {
  if (!p) return MOE_DECODE_EINVAL;
  p->timeline = on != 0;
  return MOE_DECODE_OK;
}

int moe_decode_timeline_read(moe_decode_handle p, int32_t kernel, uint64_t* h_out, size_t n, int32_t* blocks) {
  if (!p || kernel < 0 || kernel >= kKernels || !blocks) return MOE_DECODE_EINVAL;
  const int nb = p->last_grid[kernel] < kTlBlocks ? p->last_grid[kernel] : kTlBlocks;
  *blocks = nb;
  const size_t want = (size_t)nb * kTlPoints;
  if (!h_out || n < want) return MOE_DECODE_EINVAL;
  hipError_t e = hipMemcpy(h_out, p->tl_base + (size_t)kernel * kTlBlocks * kTlPoints, want * 8,
                           hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(p, e, "hipMemcpy");
  return MOE_DECODE_OK;
}

void moe_decode_destroy(moe_decode_handle p) {
  if (!p) return;
  free_timing(p);
  if (p->base) (void)hipFree(p->base);
  delete p;
}

int moe_decode_quantize_weight(const float* d_w, int32_t count, int32_t rows, int32_t cols, void* d_q,
                               void* d_scales, void* stream) {
  if (count < 1 || rows < 32 || cols < 32 || rows % 32 || cols % 32) return MOE_DECODE_EINVAL;
  if (!aligned16(d_w) || !aligned16(d_q) || d_scales == nullptr) return MOE_DECODE_EINVAL;
  hipError_t e = launch_quant_weight(d_w, count, rows, cols, static_cast<uint8_t*>(d_q),
                                     static_cast<uint8_t*>(d_scales), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(nullptr, e, "quantize launch");
  return MOE_DECODE_OK;
}

int moe_decode_quantize_weight_fp4(const float* d_w, int32_t count, int32_t rows, int32_t cols, void* d_q,
                                   void* d_scales, void* stream) {
  if (count < 1 || rows < 16 || rows % 16 || cols < 32 || cols % 32) return MOE_DECODE_EINVAL;
  if (!aligned16(d_w) || !aligned16(d_q) || d_scales == nullptr) return MOE_DECODE_EINVAL;
  hipError_t e = launch_quant_weight_fp4(d_w, count, rows, cols, static_cast<uint8_t*>(d_q),
                                         static_cast<uint8_t*>(d_scales), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(nullptr, e, "quantize launch");
  return MOE_DECODE_OK;
}

int moe_decode_read_probe(const void* d_buf, size_t bytes, uint32_t* d_sink, void* stream) {
  if (bytes < 16 || bytes % 16 || !aligned16(d_buf) || d_sink == nullptr ||
      reinterpret_cast<uintptr_t>(d_sink) % 4)
    return MOE_DECODE_EINVAL;
  hipError_t e = launch_read_probe(d_buf, bytes, d_sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(nullptr, e, "read probe launch");
  return MOE_DECODE_OK;
}

int moe_decode_hc_fold(int32_t m, int32_t hidden, const void* d_part, const void* d_residual, const float* d_post,
                       const float* d_res, const float* d_pre, void* d_residual_out, void* d_x, void* stream) {
  if (m < 1 || m > kMaxTokens || hidden < 128 || hidden > kMaxHidden || hidden % 128) return MOE_DECODE_EINVAL;
  const void* ptrs[] = {d_part, d_residual, d_post, d_res, d_pre, d_residual_out, d_x};
  for (const void* q : ptrs)
    if (!aligned16(q)) return MOE_DECODE_EINVAL;
  // the new residual may replace the old one in place, or lie apart from it;
  // x lies apart from every input
  const uintptr_t ri = reinterpret_cast<uintptr_t>(d_residual), ro = reinterpret_cast<uintptr_t>(d_residual_out);
  const uintptr_t rn = (uintptr_t)m * 4 * hidden * 2, xn = (uintptr_t)m * hidden * 2;
  if (ri != ro && ri < ro + rn && ro < ri + rn) return MOE_DECODE_EINVAL;
  const uintptr_t xo = reinterpret_cast<uintptr_t>(d_x), po = reinterpret_cast<uintptr_t>(d_part);
  if ((xo < ri + rn && ri < xo + xn) || (xo < ro + rn && ro < xo + xn) || (xo < po + xn && po < xo + xn))
    return MOE_DECODE_EINVAL;
  hipError_t e = launch_hc_fold(m, hidden, static_cast<const uint16_t*>(d_part),
                                static_cast<const uint16_t*>(d_residual), d_post, d_res, d_pre,
                                static_cast<uint16_t*>(d_residual_out), static_cast<uint16_t*>(d_x),
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(nullptr, e, "hc_fold launch");
  return MOE_DECODE_OK;
}

int moe_decode_attn_x8(int32_t m, int32_t hidden, const void* d_x, const void* d_norm_w, float rms_eps, void* d_x8,
                       void* d_x8s, void* stream) {
  if (m < 1 || m > kMaxTokens || hidden < 128 || hidden > kMaxHidden || hidden % 128) return MOE_DECODE_EINVAL;
  if (!std::isfinite(rms_eps) || rms_eps < 0.0f) return MOE_DECODE_EINVAL;
  const void* ptrs[] = {d_x, d_norm_w, d_x8, d_x8s};
  for (const void* q : ptrs)
    if (!aligned16(q)) return MOE_DECODE_EINVAL;
  hipError_t e = launch_attn_x8(m, hidden, static_cast<const uint16_t*>(d_x), static_cast<const uint16_t*>(d_norm_w),
                                rms_eps, static_cast<uint8_t*>(d_x8), static_cast<uint8_t*>(d_x8s),
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(nullptr, e, "attn_x8 launch");
  return MOE_DECODE_OK;
}

const char* moe_decode_strerror(int code) {
  switch (code) {
    case MOE_DECODE_OK: return "success";
    case MOE_DECODE_EINVAL: return "invalid argument";
    case MOE_DECODE_ENOMEM: return "out of memory";
    case MOE_DECODE_EHIP: return "HIP runtime error";
    case MOE_DECODE_ECAPTURE: return "called during stream capture";
    default: return "unknown error";
  }
}

const char* moe_decode_last_hip_error(moe_decode_handle p) { return p ? p->err.c_str() : g_last_error.c_str(); }

}  // extern "C"
