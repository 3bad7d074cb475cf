"""Benchmark of the decode MoE FFN on one MI355X.

A step is one moe_decode_run -- the whole hot path: norm + MXFP8, router,
top-k and plan, w13 + SiLU*up, w2 + weighted combine -- over one batch of M
synthetic token rows already resident in HBM.  Default workload: the
DeepSeek-V4.1-style layer at M = 1 (H 5120, 256 experts top-8, I = Is = 2048,
E4M3 weights with 32 x 32 E8M0 blocks).

The timed region replays captured HIP graphs of the step.  To keep the
256 MB last-level cache from serving the expert weights, the steps rotate over
several device copies of the whole weight set, each with its own input rows
(so each copy picks its own experts).  After the timed region a second pass of
the same steps runs eagerly with the library's HIP events around each kernel
(on the run's stream), which gives the dominant kernel's average duration for
the roofline.

Output: one JSON line (rank 0).  `python bench.py --gpus N` with N > 1 exits:
this build measures one GPU.
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


def expert_bytes(H: int, I: int) -> dict:
    """Algorithmic bytes of one expert: weights and their E8M0 codes."""
    w13 = 2 * I * H + (2 * I // 32) * (H // 32)
    w2 = H * I + (H // 32) * (I // 32)
    return {"w13": w13, "w2": w2}


def make_weights(cfg: dict, seed: int, dev):
    """One device copy of the expert weights: N(0, 0.02) fp32 drawn on the GPU,
    quantised by the library's weight quantiser (32 x 32 E8M0 blocks)."""
    import torch
    import moe_decode_layer_seam_amd as mdl

    E, H, I, Is = cfg["experts"], cfg["hidden"], cfg["inter"], cfg["shared_inter"]
    g = torch.Generator(device=dev)
    g.manual_seed(1000 + seed)
    w = {
        "w13": torch.empty((E, 2 * I, H), dtype=torch.uint8, device=dev),
        "w13_s": torch.empty((E, 2 * I // 32, H // 32), dtype=torch.uint8, device=dev),
        "w2": torch.empty((E, H, I), dtype=torch.uint8, device=dev),
        "w2_s": torch.empty((E, H // 32, I // 32), dtype=torch.uint8, device=dev),
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
            mdl.quantize_weight(f, w[name][e0:e0 + n], w[name + "_s"][e0:e0 + n])
            del f
    for name, rows, cols in (("sgu", 2 * Is, H), ("sw2", H, Is)):
        f = torch.randn((rows, cols), generator=g, device=dev, dtype=torch.float32) * 0.02
        mdl.quantize_weight(f, w[name], w[name + "_s"])
        del f
    torch.cuda.synchronize()
    return w


def cpu_baseline(cfg: dict, budget_s: float = 12.0, workers: int = 16) -> dict:
    """The oracle, single-threaded, on the same workload shape: the layer at
    M rows for seed-0 inputs, repeated until about budget_s of CPU time.  Only
    the picked experts' weights are drawn and quantised (the oracle reads no
    other expert); drawing them is setup, not timed."""
    import numpy as np
    import oracle
    import synth
    from tests import data

    m = cfg["m"]
    inp, w = data.build_layer(0, cfg, experts="picked", workers=workers)
    dims = data.dims_of(cfg)
    reps, t0 = 0, time.perf_counter()
    rows = list(range(m))
    while True:
        oracle.layer(dims, inp, w, rows=rows)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    return {"value": reps * m / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{cfg['name']}: {reps} full-layer oracle pass(es) of the M={m} "
                      f"seed-0 step, one thread, {el:.1f} s; expert weights of the picked "
                      f"experts only (drawn outside the timing)"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="workload index 1-4 (0 = tiny)")
    ap.add_argument("--copies", type=int, default=0, help="weight copies rotated (0: auto)")
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the layer runs at TP=1 on a single MI355X)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import moe_decode_layer_seam_amd as mdl
    import synth

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).cuda()

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    cfg = dict(synth.CONFIGS[args.config])
    m, H, E, K, I, Is = cfg["m"], cfg["hidden"], cfg["experts"], cfg["topk"], cfg["inter"], cfg["shared_inter"]
    eb = expert_bytes(H, I)
    ebs = expert_bytes(H, Is)
    per_step_expected = (min(E, m * K) + 1) * (eb["w13"] + eb["w2"])
    copies = args.copies or max(2, min(8, -(-2 * 512 * 2**20 // per_step_expected)))

    print(f"[bench] {cfg['name']}: building {copies} weight copies", file=sys.stderr, flush=True)
    t0 = time.time()
    wsets = [make_weights(cfg, c, dev) for c in range(copies)]
    xs = [bf16_dev(synth.to_bf16_bits(synth.normal(10 + c, synth.STREAM["x"], (m, H)))) for c in range(copies)]
    small = synth.small_inputs(0, 1, H, E)
    norm_w, gate_w = bf16_dev(small["norm_w"]), bf16_dev(small["gate_w"])
    bias = torch.from_numpy(small["bias"]).to(dev)
    outs = [torch.empty((m, H), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    print(f"[bench] weights ready in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    h = mdl.plan(H, E, K, I, Is, m, cfg["rms_eps"], cfg["routed_scale"])
    stream = torch.cuda.current_stream()

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

    graphs = []
    if args.mode == "graph":
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    step(c)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(s)
        for c in range(copies):
            graphs[c].replay()
        torch.cuda.synchronize()

    # ---- timed region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        if graphs:
            graphs[i % copies].replay()
        else:
            step(i % copies)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev0.elapsed_time(ev1)
    ms_step = ms / args.steps

    # ---- per-kernel durations: the same steps, eager, HIP events per kernel
    mdl.timing(h, True)
    for i in range(args.steps):
        step(i % copies)
    torch.cuda.synchronize()
    kern = {}
    for k in ("seam", "route", "w13", "w13_finish", "w2"):
        tot, runs = mdl.timing_read(h, k)
        kern[k] = tot / max(1, runs)
    mdl.timing(h, False)

    # algorithmic bytes of the dominant kernel (w13) per launch: every active
    # expert's gate/up weights and codes (shared expert included), the MXFP8
    # rows it reads and the MXFP8 intermediate it writes
    steps_U = [U[i % copies] for i in range(args.steps)]
    avg_U = sum(steps_U) / len(steps_U)
    w13_bytes = avg_U * eb["w13"] + ebs["w13"] + m * (H + H // 32) + (m * K + m) * (max(I, Is) + max(I, Is) // 32)
    expert_step_bytes = avg_U * (eb["w13"] + eb["w2"]) + ebs["w13"] + ebs["w2"]
    achieved = w13_bytes / (kern["w13"] * 1e-3) / 1e9

    res = {
        "metric": METRIC,
        "value": m * args.steps / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']}: M={m} token rows, hidden {H}, {E} routed experts top-{K}, "
                               f"intermediate {I}, shared expert {Is}, E4M3 weights with 32x32 E8M0 blocks",
                   "tokens": m, "mode": args.mode, "weight_copies": copies},
        "us_per_layer": ms_step * 1e3,
        "expert_hbm_frac": expert_step_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "active_experts_avg": avg_U,
        "kernel_us": {k: v * 1e3 for k, v in kern.items()},
        "wall_s": wall,
        "roofline": {"bound": "hbm", "kernel": "w13", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None},
    }
    mdl.destroy(h)
    del graphs, wsets
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
