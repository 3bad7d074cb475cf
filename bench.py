"""Benchmark of the decode MoE FFN on one MI355X.

A step is one moe_decode_run -- the whole hot path: norm + MXFP8, router,
top-k and plan, w13 + SiLU*up, w2 + weighted combine -- over one batch of M
synthetic token rows already resident in HBM.  Default workload: the
DeepSeek-V4.1-style layer at M = 1 (H 5120, 256 experts top-8, I = Is = 2048,
E4M3 weights with 32 x 32 E8M0 blocks).

The timed region replays captured HIP graphs, each holding several
consecutive steps (as a decode graph holds many layers).  To keep the 256 MB
last-level cache from serving the expert weights, the steps rotate over
several device copies of the whole weight set, each with its own input rows
(so each copy picks its own experts); a labelled cache-warm figure repeats one
copy.  Right before the timed region the steps are warmed up in the same
mode for --warmup steps and at least --warmup-s seconds, so that the GPU's
clocks have settled after the graph capture.  After the timed region the
same steps run eagerly, each kernel's dispatch recording its own start/stop
HIP events on the run's stream, which gives the dominant kernel's average
duration for the roofline.

Output: one JSON line (rank 0).  `python bench.py --gpus N` with N > 1 exits:
the benchmark measures one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE decode layer µs & tokens/s at M=1/16/48; % HBM roofline on expert weights"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def expert_bytes(H: int, I: int, fmt: str = "e4m3") -> dict:
    """Algorithmic bytes of one expert: weights and their E8M0 codes (E4M3
    with 32 x 32 blocks, or MXFP4: E2M1 pairs with a code per row and 32
    columns)."""
    if fmt == "mxfp4":
        return {"w13": 2 * I * (H // 2) + 2 * I * (H // 32), "w2": H * (I // 2) + H * (I // 32)}
    w13 = 2 * I * H + (2 * I // 32) * (H // 32)
    w2 = H * I + (H // 32) * (I // 32)
    return {"w13": w13, "w2": w2}


def w13_input_bytes(m: int, H: int, E: int, K: int) -> int:
    """Algorithmic bytes the w13 launch (or the persistent launch) reads
    besides the expert weights.  Steps of up to 4 tokens (E <= 256, H <= 8192,
    at most 64 pairs) run the seam and the router in that launch: it reads
    the bf16 rows, the norm weight, the router's gate rows and bias.
    Otherwise it reads the MXFP8 rows and their codes."""
    if m <= 4 and m * K <= 64 and E <= 256 and H <= 8192:
        return 2 * m * H + 2 * H + 2 * E * H + 4 * E
    return m * (H + H // 32)


def read_peak(gib: float = 4.0, reps: int = 5) -> dict:
    """Measured HBM read rate of a plain stream over gib GiB: the library's
    read probe (128-bit non-temporal loads, every byte once), timed with
    events on the current stream; best and median of reps launches after one
    untimed launch."""
    import torch
    import moe_decode_layer_seam_amd as mdl

    n = int(gib * 2**30) // 16 * 16
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(mdl.PROBE_BLOCKS, dtype=torch.int32, device="cuda")
    mdl.read_probe(buf, sink)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        mdl.read_probe(buf, sink)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    del buf
    torch.cuda.empty_cache()
    ts.sort()
    return {"bytes": n, "reps": reps, "gbs_best": n / (ts[0] * 1e-3) / 1e9,
            "gbs_median": n / (ts[len(ts) // 2] * 1e-3) / 1e9,
            "kernel": f"moe_decode_read_probe: 128-bit non-temporal loads, {mdl.PROBE_BLOCKS} blocks x 256 "
                      "threads, 16 loads in flight per thread, a contiguous range per block"}


def make_weights(cfg: dict, seed: int, dev):
    """One device copy of the expert weights: N(0, 0.02) fp32 drawn on the GPU,
    quantised by the library's weight quantisers (E4M3 with 32 x 32 E8M0
    blocks; routed experts as MXFP4 when cfg["routed"] == "mxfp4")."""
    import torch
    import moe_decode_layer_seam_amd as mdl

    E, H, I, Is = cfg["experts"], cfg["hidden"], cfg["inter"], cfg["shared_inter"]
    fp4 = cfg.get("routed", "e4m3") == "mxfp4"
    g = torch.Generator(device=dev)
    g.manual_seed(1000 + seed)
    if fp4:
        routed = {
            "w13": torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev),
            "w13_s": torch.empty((E,) + mdl.fp4_codes_shape(2 * I, H), dtype=torch.uint8, device=dev),
            "w2": torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev),
            "w2_s": torch.empty((E,) + mdl.fp4_codes_shape(H, I), dtype=torch.uint8, device=dev),
        }
    else:
        routed = {
            "w13": torch.empty((E, 2 * I, H), dtype=torch.uint8, device=dev),
            "w13_s": torch.empty((E, 2 * I // 32, H // 32), dtype=torch.uint8, device=dev),
            "w2": torch.empty((E, H, I), dtype=torch.uint8, device=dev),
            "w2_s": torch.empty((E, H // 32, I // 32), dtype=torch.uint8, device=dev),
        }
    w = {
        **routed,
        "sgu": torch.empty((2 * Is, H), dtype=torch.uint8, device=dev),
        "sgu_s": torch.empty((2 * Is // 32, H // 32), dtype=torch.uint8, device=dev),
        "sw2": torch.empty((H, Is), dtype=torch.uint8, device=dev),
        "sw2_s": torch.empty((H // 32, Is // 32), dtype=torch.uint8, device=dev),
    }
    per = 8  # experts drawn per chunk
    for name, rows, cols in (("w13", 2 * I, H), ("w2", H, I)):
        for e0 in range(0, E, per):
            n = min(per, E - e0)
            f = torch.randn((n, rows, cols), generator=g, device=dev, dtype=torch.float32) * 0.02
            quant = mdl.quantize_weight_fp4 if fp4 else mdl.quantize_weight
            quant(f, w[name][e0:e0 + n], w[name + "_s"][e0:e0 + n])
            del f
    for name, rows, cols in (("sgu", 2 * Is, H), ("sw2", H, Is)):
        f = torch.randn((rows, cols), generator=g, device=dev, dtype=torch.float32) * 0.02
        mdl.quantize_weight(f, w[name], w[name + "_s"])
        del f
    torch.cuda.synchronize()
    return w


def cpu_baseline(cfg: dict, budget_s: float = 8.0, workers: int = 16) -> dict:
    """The oracle, single-threaded, on a bounded sample of the same workload:
    the seed-0 step's token rows one at a time (the oracle's cost is per
    token), cycling through the M rows until about budget_s of CPU time.
    Only the sampled rows' picked experts' weights are drawn and quantised
    (the oracle reads no other expert); drawing them is setup, not timed."""
    import numpy as np
    import oracle
    import synth
    from tests import data

    m, H, E = cfg["m"], cfg["hidden"], cfg["experts"]
    inp = synth.small_inputs(0, m, H, E)
    y = oracle.rmsnorm(inp["x"], inp["norm_w"], cfg["rms_eps"])
    ids = oracle.router(y, inp["gate_w"], inp["bias"], cfg["topk"], cfg["routed_scale"])["ids"]
    w = data.alloc_weights(cfg)
    filled = set()
    aff = None
    try:  # one host core, like the single-threaded oracle it times
        aff = os.sched_getaffinity(0)
    except (AttributeError, OSError):
        pass
    dims = data.dims_of(cfg)
    rows, el = 0, 0.0
    while el < budget_s and rows < 1000:
        r = rows % m
        need = set(int(e) for e in ids[r]) - filled
        if need:
            if aff:
                os.sched_setaffinity(0, aff)
            data.fill_weights(0, cfg, w, need, workers)
            filled |= need
        if aff:
            os.sched_setaffinity(0, {min(aff)})
        t0 = time.perf_counter()
        oracle.layer(dims, inp, w, rows=[r])
        el += time.perf_counter() - t0
        rows += 1
    if aff:
        os.sched_setaffinity(0, aff)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": rows / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "host_cpu": cpu, "host_nproc": os.cpu_count(),
            "sample": f"{cfg['name']}: {rows} token row(s) of the M={m} seed-0 step "
                      f"(rows 0..{min(rows, m) - 1}, one at a time), one thread, {el:.1f} s of oracle "
                      f"time; expert weights of the sampled rows' picks only (drawn outside the timing)"}


def kernel_source_hash() -> str:
    """sha256 over the sources the expert kernels are built from: the traffic
    figures measured with hardware counters hold only for this code."""
    import hashlib
    hsh = hashlib.sha256()
    for f in ("experts.hip", "route.hpp", "device.hpp", "kernels.hpp"):
        with open(os.path.join(ROOT, "moe_decode_layer_seam_amd", "csrc", f), "rb") as fh:
            hsh.update(fh.read())
    return hsh.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the counter summary under
    profiles/ (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
    calibration), or None when there is none for this workload or the kernel
    sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic_json: "):
                rec = json.loads(line[len("traffic_json: "):])
                if rec.get("kernel_src_sha256") == kernel_source_hash():
                    return rec["bytes_per_launch"]
    return None


def seam_timing(m: int, H: int, reps: int = 50) -> dict:
    """Device time of the seam upstream of the MoE at m rows of H columns:
    the hyper-connection residual fold and the attention seam's MXFP8, each
    replayed from a graph of `reps` launches on synthetic inputs resident in
    HBM.  Bytes are the algorithmic ones (every input read once, every output
    written once)."""
    import torch
    import moe_decode_layer_seam_amd as mdl
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    part = torch.randn((m, H), generator=g, device="cuda").to(torch.bfloat16)
    resid = torch.randn((m, 4, H), generator=g, device="cuda").to(torch.bfloat16)
    post = torch.rand((m, 4), generator=g, device="cuda") * 2
    res = torch.rand((m, 4, 4), generator=g, device="cuda")
    pre = torch.rand((m, 4), generator=g, device="cuda")
    rout, x = torch.empty_like(resid), torch.empty_like(part)
    norm_w = (1 + 0.1 * torch.randn((H,), generator=g, device="cuda")).to(torch.bfloat16)
    x8 = torch.empty((m, H), dtype=torch.uint8, device="cuda")
    x8s = torch.empty((m, H // 32), dtype=torch.uint8, device="cuda")
    calls = {
        "hc_fold": (lambda: mdl.hc_fold(part, resid, post, res, pre, rout, x),
                    20 * m * H + m * 24 * 4),
        "attn_x8": (lambda: mdl.attn_x8(part, norm_w, 1e-6, x8, x8s),
                    2 * m * H + 2 * H + m * H + m * H // 32),
    }
    out = {}
    for name, (fn, nbytes) in calls.items():
        fn()
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(gr, stream=s):
                for _ in range(reps):
                    fn()
        torch.cuda.current_stream().wait_stream(s)
        gr.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (5 * reps)
        out[name] = {"us": us, "bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9}
        del gr
    return out


def copy_probe(mib: int, reps: int = 5) -> int:
    """A plain device copy of known size (for calibrating the HBM byte
    counters): dst = ~src over mib MiB of int32, reps times."""
    import torch
    n = mib * 2**20 // 4
    src = torch.arange(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_mib": mib, "reps": reps, "bytes_read_per_launch": n * 4,
                      "bytes_written_per_launch": n * 4}), flush=True)
    return 0


class InvalidRun(RuntimeError):
    """A wait inside a launch timed out during the measured steps: their
    output, and so their time, is not valid."""


def auto_copies(cfg: dict, fmt: str) -> int:
    """Weight copies rotated so that the rotation's expert bytes exceed 1 GiB
    (four times the 256 MB last-level cache), 2 to 32."""
    eb = expert_bytes(cfg["hidden"], cfg["inter"], fmt)
    per_step = (min(cfg["experts"], cfg["m"] * cfg["topk"]) + 1) * (eb["w13"] + eb["w2"])
    return max(2, min(32, -(-2 * 512 * 2**20 // per_step)))


def bench_config(cfg: dict, args, wsets: list, xs_all: list, small: dict) -> dict:
    """Times one workload: K steps of graph-replayed moe_decode_run over the
    weight copies, then the same steps eagerly with per-kernel events.
    Returns the workload's block of the JSON line."""
    import numpy as np
    import torch
    import moe_decode_layer_seam_amd as mdl

    routed = args.routed
    m, H, E, K, I, Is = cfg["m"], cfg["hidden"], cfg["experts"], cfg["topk"], cfg["inter"], cfg["shared_inter"]
    copies = len(wsets)
    dev = torch.device("cuda", 0)
    eb = expert_bytes(H, I, routed)
    ebs = expert_bytes(H, Is)
    xs = [x[:m].contiguous() for x in xs_all]
    outs = [torch.empty((m, H), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    norm_w, gate_w, bias = small["norm_w"], small["gate_w"], small["bias"]

    # the plan a caller makes for this decode width
    h = mdl.plan(H, E, K, I, Is, m, cfg["rms_eps"], cfg["routed_scale"], routed=routed,
                 schedule=args.schedule)
    try:
        def step(c):
            w = wsets[c]
            mdl.run(h, cfg, xs[c], norm_w, gate_w, bias, w["w13"], w["w13_s"], w["w2"], w["w2_s"],
                    w["sgu"], w["sgu_s"], w["sw2"], w["sw2_s"], outs[c])

        # distinct routed experts of each copy's step (from the plan's counts)
        U = []
        for c in range(copies):
            step(c)
            torch.cuda.synchronize()
            U.append(int((mdl.inspect_tensor(h, "counts", torch.int32) > 0).sum().item()))
        for i in range(args.warmup):
            step(i % copies)
        torch.cuda.synchronize()
        if mdl.status(h):
            raise InvalidRun(f"{cfg['name']}: a wait timed out in the warm-up steps")

        # graphs of G consecutive steps (whole laps over the weight copies), as
        # a decode graph holds many layers; another takes the rest of a batch
        G = copies * max(1, -(-8 // copies))
        nb = 5 if args.steps >= 5 * G else 1
        sizes = [args.steps // nb + (1 if b < args.steps % nb else 0) for b in range(nb)]
        graphs = {}
        if args.mode == "graph":
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                for n in sorted(({G} | {sz % G for sz in sizes}) - {0}):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=st):
                        for i in range(n):
                            step(i % copies)
                    graphs[n] = g
            torch.cuda.current_stream().wait_stream(st)
            for g in graphs.values():
                g.replay()
            torch.cuda.synchronize()

        def run_steps(n):
            if graphs:
                for _ in range(n // G):
                    graphs[G].replay()
                if n % G:
                    graphs[n % G].replay()
            else:
                for i in range(n):
                    step(i % copies)

        # warm-up in the timed mode, right before the timed region: the
        # --warmup steps, extended to --warmup-s seconds of steps.  The GPU's
        # clocks drop while the host captures the graphs; timed right after,
        # one token ran 61.9-63.6 us a step and the draft layer 193 us, against
        # 60.0-60.9 and 186.6 us once they had settled (a second of steps;
        # three seconds gave the same)
        t_wu = time.perf_counter()
        wu_steps = 0
        chunk = 8 * (G if graphs else copies)
        while wu_steps < args.warmup or time.perf_counter() - t_wu < args.warmup_s:
            run_steps(chunk)
            wu_steps += chunk
            torch.cuda.synchronize()
        wu_s = time.perf_counter() - t_wu
        if mdl.status(h):
            raise InvalidRun(f"{cfg['name']}: a wait timed out in the warm-up replays")

        # ---- timed region
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        evs[0].record()
        for b in range(nb):
            run_steps(sizes[b])
            evs[b + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms = evs[0].elapsed_time(evs[nb])
        ms_step = ms / args.steps
        batch_us = sorted(evs[b].elapsed_time(evs[b + 1]) / sizes[b] * 1e3 for b in range(nb))
        # every timed step was valid: no wait inside a launch gave up
        st_word = mdl.status(h)
        if st_word:
            raise InvalidRun(f"{cfg['name']}: status {st_word} after the timed steps")

        # ---- cache-warm figure (labelled, not the metric): one weight copy only
        warm_us = None
        if graphs:
            gw = torch.cuda.CUDAGraph()
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                with torch.cuda.graph(gw, stream=st):
                    for i in range(G):
                        step(0)
            torch.cuda.current_stream().wait_stream(st)
            t_w = time.perf_counter()
            while time.perf_counter() - t_w < args.warmup_s:  # as before the timed region
                for _ in range(8):
                    gw.replay()
                torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(1, args.steps // G)
            e0.record()
            for _ in range(reps):
                gw.replay()
            e1.record()
            torch.cuda.synchronize()
            warm_us = e0.elapsed_time(e1) / (reps * G) * 1e3
            del gw
        graphs.clear()

        # ---- per-kernel durations: the same steps, eager, each kernel's
        # dispatch recording its own start/stop HIP events (on the run's stream)
        mdl.timing(h, True)
        for i in range(args.steps):
            step(i % copies)
        torch.cuda.synchronize()
        kern = {}
        for k in mdl.KERNELS:
            tot, runs = mdl.timing_read(h, k)
            if runs:
                kern[k] = tot / runs
        mdl.timing(h, False)
        st_word = mdl.status(h)
        if st_word:
            raise InvalidRun(f"{cfg['name']}: status {st_word} after the per-kernel timing steps")

        # MFMA row occupancy: useful token rows / issued 16-row tiles (last copy)
        counts = mdl.inspect_tensor(h, "counts", torch.int32).cpu().numpy()
    finally:
        mdl.destroy(h)
    tiles = int(sum(-(-int(c) // 16) for c in counts if c > 0)) + -(-m // 16)
    row_occupancy = (m * K + m) / (16 * tiles)

    # algorithmic bytes per launch of the dominant kernel (the persistent
    # launch where it ran, else w13): every active expert's weights and codes
    # (shared expert included) and the rows they are multiplied with (MXFP8,
    # or at m <= 4 the bf16 rows, norm weight and router weights the launch's
    # own seam and router read); w2 also reads the SiLU*up intermediate,
    # which the persistent launch makes itself
    steps_U = [U[i % copies] for i in range(args.steps)]
    avg_U = sum(steps_U) / len(steps_U)
    w13_bytes = avg_U * eb["w13"] + ebs["w13"] + w13_input_bytes(m, H, E, K)
    expert_step_bytes = avg_U * (eb["w13"] + eb["w2"]) + ebs["w13"] + ebs["w2"]
    a8_bytes = (m * K + m) * (max(I, Is) + max(I, Is) // 32)
    w2_bytes = avg_U * eb["w2"] + ebs["w2"] + a8_bytes
    if "persistent" in kern:
        dom, dom_bytes = "persistent", w13_bytes + w2_bytes - a8_bytes
        kernel_gbs = {"persistent": dom_bytes / (kern["persistent"] * 1e-3) / 1e9}
    else:
        dom, dom_bytes = "w13", w13_bytes
        kernel_gbs = {"w13": w13_bytes / (kern["w13"] * 1e-3) / 1e9,
                      "w2": w2_bytes / (kern["w2"] * 1e-3) / 1e9}
    achieved = kernel_gbs[dom]
    workload = cfg["name"] + ("" if routed == "e4m3" else "_mxfp4")
    return {
        "workload": f"{cfg['name']}: M={m} token rows, hidden {H}, {E} routed experts top-{K}, "
                    f"intermediate {I}, shared expert {Is}, " + (
                        "E4M3 weights with 32x32 E8M0 blocks" if routed == "e4m3" else
                        "routed experts MXFP4 (E2M1, 1x32 E8M0), shared expert E4M3 32x32"),
        "tokens": m,
        "us_per_layer": ms_step * 1e3,
        "tokens_per_s": m * args.steps / (ms * 1e-3),
        "ms_per_step": ms_step,
        "batch_us_per_layer": batch_us,
        "median_batch_us_per_layer": batch_us[len(batch_us) // 2],
        "cache_warm_us_per_layer": warm_us,
        "steps_per_graph": G if args.mode == "graph" else None,
        "warmup_steps": wu_steps,
        "warmup_s": wu_s,
        "weight_copies": copies,
        "mfma_row_occupancy": row_occupancy,
        "expert_hbm_frac": expert_step_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "expert_step_bytes": expert_step_bytes,
        "active_experts_avg": avg_U,
        "kernel_us": {k: v * 1e3 for k, v in kern.items()},
        "kernel_gbs": kernel_gbs,
        "status": 0,
        "wall_s": wall,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(dom, workload),
                     "algorithmic_bytes": dom_bytes},
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warmup-s", type=float, default=1.0,
                    help="warm-up before each timed region lasts at least this long (seconds)")
    ap.add_argument("--configs", default="1,2,3,4",
                    help="workload indices, the first one the headline (0 tiny; 1-3 the layer at "
                         "M = 1, 16, 48; 4 the draft layer; 5-6 the eight-way tensor-parallel share)")
    ap.add_argument("--config", type=int, default=None, help="a single workload (same as --configs N)")
    ap.add_argument("--copies", type=int, default=0, help="weight copies rotated (0: auto)")
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=8.0, help="oracle seconds per workload")
    ap.add_argument("--routed", choices=("e4m3", "mxfp4"), default="e4m3",
                    help="routed experts' weight format (the shared expert is E4M3)")
    ap.add_argument("--schedule", choices=("auto", "launches", "persistent"), default="auto",
                    help="auto: the library's fastest (the short launches); launches: the short "
                         "launches for every step; persistent: the persistent launch for the small "
                         "steps it covers")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the upstream-seam timing and the read probe")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.copy_probe:
        return copy_probe(args.copy_probe)

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the layer runs at TP=1 on a single MI355X)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import synth

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).cuda()

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    idxs = [args.config] if args.config is not None else [int(c) for c in args.configs.split(",")]
    cfgs = [dict(synth.WORKLOADS[i], routed=args.routed) for i in idxs]

    # workloads with the same weight shapes share one set of weight copies
    blocks = {}
    done = set()
    for ci, cfg in enumerate(cfgs):
        if ci in done:
            continue
        shape = (cfg["hidden"], cfg["experts"], cfg["inter"], cfg["shared_inter"])
        group = [cj for cj, c in enumerate(cfgs)
                 if (c["hidden"], c["experts"], c["inter"], c["shared_inter"]) == shape]
        copies = args.copies or max(auto_copies(cfgs[cj], args.routed) for cj in group)
        mmax = max(cfgs[cj]["m"] for cj in group)
        print(f"[bench] {', '.join(cfgs[cj]['name'] for cj in group)}: building {copies} weight copies",
              file=sys.stderr, flush=True)
        t0 = time.time()
        wsets = [make_weights(cfg, c, dev) for c in range(copies)]
        xs_all = [bf16_dev(synth.to_bf16_bits(synth.normal(10 + c, synth.STREAM["x"], (mmax, cfg["hidden"]))))
                  for c in range(copies)]
        sm = synth.small_inputs(0, 1, cfg["hidden"], cfg["experts"])
        small = {"norm_w": bf16_dev(sm["norm_w"]), "gate_w": bf16_dev(sm["gate_w"]),
                 "bias": torch.from_numpy(sm["bias"]).to(dev)}
        print(f"[bench] weights ready in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
        for cj in group:
            print(f"[bench] timing {cfgs[cj]['name']}", file=sys.stderr, flush=True)
            try:
                blocks[cj] = bench_config(cfgs[cj], args, wsets, xs_all, small)
            except InvalidRun as e:
                print(f"[bench] INVALID RUN: {e}", file=sys.stderr, flush=True)
                return 3
            b = blocks[cj]
            print(f"[bench] {cfgs[cj]['name']}: {b['us_per_layer']:.1f} us/layer, "
                  f"expert HBM fraction {b['expert_hbm_frac']:.3f}", file=sys.stderr, flush=True)
            if cfgs[cj]["m"] <= 4 and args.schedule == "auto" and args.routed == "e4m3" and not args.no_extras:
                # labelled beside the metric: the same steps on the persistent
                # schedule (where the plan finds the launch applicable)
                pargs = argparse.Namespace(**vars(args))
                pargs.schedule = "persistent"
                try:
                    pb = bench_config(cfgs[cj], pargs, wsets, xs_all, small)
                except InvalidRun as e:
                    print(f"[bench] INVALID RUN: {e}", file=sys.stderr, flush=True)
                    return 3
                b["persistent_schedule"] = {
                    "launched": "persistent" in pb["kernel_us"],
                    "us_per_layer": pb["us_per_layer"], "tokens_per_s": pb["tokens_per_s"],
                    "expert_hbm_frac": pb["expert_hbm_frac"], "kernel_us": pb["kernel_us"],
                    "status": pb["status"]}
                print(f"[bench] {cfgs[cj]['name']} on the persistent schedule: {pb['us_per_layer']:.1f} us/layer",
                      file=sys.stderr, flush=True)
            done.add(cj)
        del wsets, xs_all, small
        torch.cuda.empty_cache()

    head_cfg, head = cfgs[0], blocks[0]
    res = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3" if args.routed == "e4m3" else "e4m3 x e2m1 (routed), e4m3 (shared)",
        "data": "synthetic",
        "config": {"workload": head["workload"], "tokens": head["tokens"], "mode": args.mode,
                   "weight_copies": head["weight_copies"], "schedule": args.schedule},
        "us_per_layer": head["us_per_layer"],
        "expert_hbm_frac": head["expert_hbm_frac"],
        "roofline": head["roofline"],
        "kernel_us": head["kernel_us"],
        "status": 0,
        "configs": {c["name"]: blocks[i] for i, c in enumerate(cfgs)},
    }
    if not args.no_extras:
        # the seam upstream of the MoE (reported beside the step, not part of it)
        res["upstream_seam"] = {f"m{mm}": seam_timing(mm, head_cfg["hidden"]) for mm in (1, 48)}
        # the measured streaming-read peak beside the published one
        res["hbm_read_probe"] = read_peak()
        for b in res["configs"].values():
            b["expert_hbm_frac_of_measured"] = (b["expert_step_bytes"] / (b["ms_per_step"] * 1e-3)
                                                / (res["hbm_read_probe"]["gbs_best"] * 1e9))
    if not args.no_cpu_baseline:
        for i, c in enumerate(cfgs):
            print(f"[bench] timing the oracle on the host: {c['name']}", file=sys.stderr, flush=True)
            blocks[i]["cpu_baseline"] = cpu_baseline(c, args.cpu_budget)
        res["cpu_baseline"] = blocks[0]["cpu_baseline"]
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
