"""An independent reference of the layer built from torch library primitives
(fp8 and bf16 casts, float64 matmul, sigmoid, topk) for tiny shapes.  FP4
(E2M1) weights, which torch cannot cast, are decoded through the golden table
tests/golden/e2m1_values.txt.

It shares nothing with the oracle: it exists to pin the oracle's expert path,
router and combine against a second implementation whose number-format
handling is torch's own.  Float64 throughout; the fp32 and bf16 roundings the
method defines are torch casts.
"""
from __future__ import annotations

import os

import numpy as np
import torch

F64 = torch.float64


def _e2m1_table() -> torch.Tensor:
    vals = [0.0] * 16
    with open(os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                nib, v = line.split()
                vals[int(nib, 16)] = float(v)
    return torch.tensor(vals, dtype=F64)


E2M1 = _e2m1_table()


def bf16_bits_to_f64(bits) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(F64)


def e4m3_to_f64(b) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(b, np.uint8))
    return t.view(torch.float8_e4m3fn).to(F64)


def code_of(amax: torch.Tensor) -> torch.Tensor:
    """clamp(ceil(log2(max(amax, FLT_MIN) / 448)) + 127, 0, 254)."""
    a = torch.clamp(amax, min=2.0 ** -126)
    return torch.clamp(torch.ceil(torch.log2(a / 448.0)) + 127, 0, 254)


def mx_quant(v: torch.Tensor):
    """Row-wise MXFP8 (last dim, 32-groups): (E4M3 bytes, codes), via torch's
    float8_e4m3fn cast (round to nearest even)."""
    g = v.reshape(*v.shape[:-1], -1, 32)
    code = code_of(g.abs().amax(-1))
    s = torch.clamp(g * torch.exp2(127 - code)[..., None], -448, 448)
    q = s.to(torch.float8_e4m3fn).view(torch.uint8).reshape(v.shape)
    return q, code.to(torch.uint8)


def mx_dequant(q: torch.Tensor, code: torch.Tensor) -> torch.Tensor:
    v = q.view(torch.float8_e4m3fn).to(F64)
    g = v.reshape(*v.shape[:-1], -1, 32)
    return (g * torch.exp2(code.to(F64) - 127)[..., None]).reshape(v.shape)


def block_dequant(q, s) -> torch.Tensor:
    """[N, K] E4M3 with [N/32, K/32] block codes -> float64."""
    v = e4m3_to_f64(q)
    sc = torch.from_numpy(np.ascontiguousarray(s, np.uint8)).to(F64)
    sc = sc.repeat_interleave(32, 0).repeat_interleave(32, 1)
    return v * torch.exp2(sc - 127)


def fp4_dequant(q, s) -> torch.Tensor:
    """[N, K/2] E2M1 pairs (column 2i in the low nibble) with blocked codes
    [N/16, ceil(K/512), 16, 16] (tile of 16 rows, 512-column segment, row,
    32-column block) -> float64 [N, K]."""
    b = torch.from_numpy(np.ascontiguousarray(q, np.uint8)).to(torch.int64)
    v = torch.stack([E2M1[b & 0xF], E2M1[b >> 4]], dim=-1).reshape(b.shape[0], -1)
    N, K = v.shape
    c = torch.from_numpy(np.ascontiguousarray(s, np.uint8)).to(F64)  # [N/16, nsg, 16, 16]
    c = c.permute(0, 2, 1, 3).reshape(N, -1)[:, :K // 32]           # [N, K/32]
    return v * torch.exp2(c.repeat_interleave(32, 1) - 127)


def dequant(q, s, fmt: str) -> torch.Tensor:
    return fp4_dequant(q, s) if fmt == "mxfp4" else block_dequant(q, s)


def expert(xq, xc, w13, w13_s, w2, w2_s, fmt: str = "e4m3"):
    """One token through one expert: (y [H] f64, a8 [I] u8, a8s [I/32] u8)."""
    xd = mx_dequant(xq, xc)
    h = dequant(w13, w13_s, fmt) @ xd
    inter = h.shape[0] // 2
    a = (torch.nn.functional.silu(h[:inter]) * h[inter:]).to(torch.float32).to(F64)
    aq, ac = mx_quant(a)
    y = dequant(w2, w2_s, fmt) @ mx_dequant(aq, ac)
    return y, aq, ac


def layer(dims: dict, inp: dict, w: dict, y_bits) -> dict:
    """Router, experts and combine on the given normed bf16 rows y_bits."""
    E, K = dims["experts"], dims["topk"]
    y = bf16_bits_to_f64(y_bits)
    xq, xc = mx_quant(y)
    G = bf16_bits_to_f64(inp["gate_w"])
    logits = y @ G.T
    s = torch.sigmoid(logits)
    b = s + torch.from_numpy(np.asarray(inp["bias"], np.float32)).to(F64)
    top = torch.topk(b, K, dim=-1, largest=True, sorted=True)
    ids = top.indices
    ssel = torch.gather(s, 1, ids)
    wts = dims.get("routed_scale", 1.0) * ssel / ssel.sum(-1, keepdim=True)
    m, H = y.shape
    out = torch.zeros(m, H, dtype=F64)
    for t in range(m):
        for j in range(K):
            e = int(ids[t, j])
            ye, _, _ = expert(xq[t], xc[t], w["w13"][e], w["w13_s"][e], w["w2"][e], w["w2_s"][e],
                              dims.get("routed", "e4m3"))
            out[t] += wts[t, j] * ye
        ys, _, _ = expert(xq[t], xc[t], w["sgu"], w["sgu_s"], w["sw2"], w["sw2_s"])
        out[t] += ys
    return {"x8": xq.numpy(), "x8s": xc.numpy(), "logits": logits.numpy(),
            "ids": ids.numpy().astype(np.int32), "wts": wts.numpy(),
            "out_f64": out.numpy()}
