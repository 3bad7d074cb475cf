"""Test inputs: seeded draws from ``synth`` with the expert weights quantised
by the oracle's quantisers: E4M3 with 32 x 32 E8M0 blocks, or, for routed
experts of a config with ``routed="mxfp4"``, E2M1 pairs with one E8M0 code
per row and 32 columns.

Weights of experts no token picks are never read by either side, so a layer
can be built with only the picked experts' weights drawn (the rest of the
weight tensors stay zero): ``experts="picked"``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth

WORKERS = max(1, min(16, os.cpu_count() or 1))


def routed_of(cfg: dict) -> str:
    return cfg.get("routed", "e4m3")


def dims_of(cfg: dict) -> dict:
    d = {k: cfg[k] for k in ("hidden", "experts", "topk", "inter",
                             "shared_inter", "rms_eps", "routed_scale")}
    d["routed"] = routed_of(cfg)
    return d


def alloc_weights(cfg: dict) -> dict:
    E, H, I, Is = cfg["experts"], cfg["hidden"], cfg["inter"], cfg["shared_inter"]
    if routed_of(cfg) == "mxfp4":
        routed = {
            "w13": np.zeros((E, 2 * I, H // 2), np.uint8),
            "w13_s": np.zeros((E,) + oracle.fp4_codes_shape(2 * I, H), np.uint8),
            "w2": np.zeros((E, H, I // 2), np.uint8),
            "w2_s": np.zeros((E,) + oracle.fp4_codes_shape(H, I), np.uint8),
        }
    else:
        routed = {
            "w13": np.zeros((E, 2 * I, H), np.uint8),
            "w13_s": np.zeros((E, 2 * I // 32, H // 32), np.uint8),
            "w2": np.zeros((E, H, I), np.uint8),
            "w2_s": np.zeros((E, H // 32, I // 32), np.uint8),
        }
    return {
        **routed,
        "sgu": np.zeros((2 * Is, H), np.uint8),
        "sgu_s": np.zeros((2 * Is // 32, H // 32), np.uint8),
        "sw2": np.zeros((H, Is), np.uint8),
        "sw2_s": np.zeros((H // 32, Is // 32), np.uint8),
    }


def fill_weights(seed: int, cfg: dict, w: dict, experts, workers: int = WORKERS) -> None:
    """Draw and quantise the given routed experts' weights (and the shared
    expert's) into ``w`` in place."""
    H, I, Is = cfg["hidden"], cfg["inter"], cfg["shared_inter"]
    rq = oracle.quant_weight_fp4_into if routed_of(cfg) == "mxfp4" else oracle.quant_weight_into

    def one(job):
        name, e = job
        if name == "w13":
            rq(synth.expert_f32(seed, "w13", e, 2 * I, H), w["w13"][e], w["w13_s"][e])
        elif name == "w2":
            rq(synth.expert_f32(seed, "w2", e, H, I), w["w2"][e], w["w2_s"][e])
        elif name == "sgu":
            oracle.quant_weight_into(synth.expert_f32(seed, "sgu", 0, 2 * Is, H),
                                     w["sgu"], w["sgu_s"])
        else:
            oracle.quant_weight_into(synth.expert_f32(seed, "sw2", 0, H, Is),
                                     w["sw2"], w["sw2_s"])

    jobs = [("sgu", 0), ("sw2", 0)]
    for e in sorted(set(int(e) for e in experts)):
        jobs += [("w13", e), ("w2", e)]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, jobs))


def build_layer(seed: int, cfg: dict, m: int | None = None, experts="all",
                workers: int = WORKERS) -> tuple[dict, dict]:
    """(inputs, weights) of one layer.  experts: "all", "picked" (only the
    experts the oracle's router picks for these m rows) or an iterable."""
    m = cfg["m"] if m is None else m
    inp = synth.small_inputs(seed, m, cfg["hidden"], cfg["experts"])
    w = alloc_weights(cfg)
    if isinstance(experts, str) and experts == "all":
        experts = range(cfg["experts"])
    elif isinstance(experts, str) and experts == "picked":
        y = oracle.rmsnorm(inp["x"], inp["norm_w"], cfg["rms_eps"])
        experts = np.unique(oracle.router(y, inp["gate_w"], inp["bias"],
                                          cfg["topk"], cfg["routed_scale"])["ids"])
    fill_weights(seed, cfg, w, experts, workers)
    return inp, w
