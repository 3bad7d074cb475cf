"""Helpers of the GPU tests: move seeded layer inputs to the device, run the
library through its C ABI, read its intermediates back, compare with the
oracle."""
from __future__ import annotations

import numpy as np
import torch

import moe_decode_layer_seam_amd as mdl

WEIGHT_NAMES = ("w13", "w13_s", "w2", "w2_s", "sgu", "sgu_s", "sw2", "sw2_s")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()


def weights_dev(w: dict) -> dict:
    return {n: u8_dev(w[n]) for n in WEIGHT_NAMES}


def inputs_dev(inp: dict) -> dict:
    return {"x": bf16_dev(inp["x"]), "norm_w": bf16_dev(inp["norm_w"]),
            "gate_w": bf16_dev(inp["gate_w"]),
            "bias": torch.from_numpy(np.ascontiguousarray(inp["bias"], np.float32)).cuda()}


def run(handle, dims, dinp, dw, x=None, out=None) -> torch.Tensor:
    x = dinp["x"] if x is None else x
    if out is None:
        out = torch.empty_like(x)
    mdl.run(handle, dims, x, dinp["norm_w"], dinp["gate_w"], dinp["bias"],
            dw["w13"], dw["w13_s"], dw["w2"], dw["w2_s"], dw["sgu"], dw["sgu_s"],
            dw["sw2"], dw["sw2_s"], out)
    return out


def tap(handle, name: str, dtype=torch.uint8) -> np.ndarray:
    return mdl.inspect_tensor(handle, name, dtype).cpu().numpy()


def out_f64(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)


def assert_out_close(got: np.ndarray, ref: np.ndarray, what: str = "out") -> None:
    """bf16 output bar: |gpu - ref| <= 1e-2 + 2e-2 |ref| element by element."""
    err = np.abs(got - ref)
    bound = 1e-2 + 2e-2 * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
        f"worst |d|={err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}")
