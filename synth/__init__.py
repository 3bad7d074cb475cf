"""Seeded synthetic inputs for the decode MoE FFN.

The one module both sides read their inputs from: the CPU oracle (through the
tests) and the HIP path (through the tests, the smoke check and the
benchmark).  It holds none of the layer's arithmetic -- it draws normal
samples from a counter-based generator (``synth.c``) and rounds the
activation-like tensors to bf16, which is how those tensors are defined.
The expert weights come out as fp32 draws; quantising them is the caller's
business (the oracle's quantiser in the tests, the library's in the bench).

Recipe (one stream per tensor, element index = flat row-major index, so a
slice of a tensor, e.g. one expert, can be drawn on its own):

  x       [M, H]  bf16  N(0, 1)              stream 1
  norm_w  [H]     bf16  1 + N(0, 0.1)        stream 2
  gate_w  [E, H]  bf16  N(0, 0.02)           stream 3
  bias    [E]     f32   N(0, 0.01)           stream 4
  w13     [E, 2I, H]    N(0, 0.02) fp32      stream 5
  w2      [E, H, I]     N(0, 0.02) fp32      stream 6
  sgu     [2Is, H]      N(0, 0.02) fp32      stream 7
  sw2     [H, Is]       N(0, 0.02) fp32      stream 8
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")

STREAM = {"x": 1, "norm_w": 2, "gate_w": 3, "bias": 4,
          "w13": 5, "w2": 6, "sgu": 7, "sw2": 8}


def build() -> str:
    """Compile the generator (gcc); returns the library path."""
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-o", _SO,
           os.path.join(_HERE, "synth.c"), "-lm"]
    subprocess.check_call(cmd)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        lib.synth_normal_f32.argtypes = [
            ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
            ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        lib.synth_normal_f32.restype = None
        _lib = lib
    return _lib


def normal(seed: int, stream: int, shape, mean: float = 0.0, std: float = 1.0,
           start: int = 0) -> np.ndarray:
    """fp32 draws of N(mean, std) for flat indices [start, start + prod(shape))."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_f32(seed, stream, start, n, mean, std,
                             out.ctypes.data)
    return out.reshape(shape)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even.

    Uses torch's conversion: defining an input tensor as bf16 is part of the
    input recipe, not of the layer's arithmetic."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def small_inputs(seed: int, m: int, hidden: int, experts: int) -> dict:
    """x, norm_w, gate_w (bf16 bit patterns) and bias (fp32) of one layer."""
    return {
        "x": to_bf16_bits(normal(seed, STREAM["x"], (m, hidden))),
        "norm_w": to_bf16_bits(normal(seed, STREAM["norm_w"], (hidden,), 1.0, 0.1)),
        "gate_w": to_bf16_bits(normal(seed, STREAM["gate_w"], (experts, hidden), 0.0, 0.02)),
        "bias": normal(seed, STREAM["bias"], (experts,), 0.0, 0.01),
    }


def expert_f32(seed: int, name: str, expert: int, rows: int, cols: int,
               std: float = 0.02) -> np.ndarray:
    """fp32 draws of one expert's [rows, cols] slice of tensor ``name``
    (for the shared-expert tensors pass expert=0)."""
    n = rows * cols
    return normal(seed, STREAM[name], (rows, cols), 0.0, std, start=expert * n)


# The workloads (shapes only).  Index 0 is the tiny layer the oracle finishes
# in well under a second; 1-3 are one DeepSeek-V4.1-style layer at 1, 16 and
# 48 token rows; 4 is the 64-expert draft layer at 48 rows; 5-6 are one GPU's
# share of layers 1 and 3 under eight-way tensor parallelism (the routed and
# shared intermediate split eight ways, hidden and router whole).
WORKLOADS = {
    0: dict(name="tiny", m=1, hidden=256, experts=8, topk=2, inter=128, shared_inter=128),
    1: dict(name="dsv41_m1", m=1, hidden=5120, experts=256, topk=8, inter=2048, shared_inter=2048),
    2: dict(name="dsv41_m16", m=16, hidden=5120, experts=256, topk=8, inter=2048, shared_inter=2048),
    3: dict(name="dsv41_m48", m=48, hidden=5120, experts=256, topk=8, inter=2048, shared_inter=2048),
    4: dict(name="draft_m48", m=48, hidden=5120, experts=64, topk=4, inter=1024, shared_inter=1024),
    5: dict(name="dsv41_tp8_m1", m=1, hidden=5120, experts=256, topk=8, inter=256, shared_inter=256),
    6: dict(name="dsv41_tp8_m48", m=48, hidden=5120, experts=256, topk=8, inter=256, shared_inter=256),
}
for _c in WORKLOADS.values():
    _c.setdefault("rms_eps", 1e-6)
    _c.setdefault("routed_scale", 1.0)
