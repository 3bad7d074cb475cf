"""The entry point for callers that cannot allocate, moe_decode_run_noalloc,
against moe_decode_run on the same inputs: the same kernels on a plan-less
scratch, so the same output bits.  Two calls in a row on one GPU, the second
with fewer token rows (and, at m <= 4, the path that routes inside the w13
launch), then a step whose scratch exceeds the array."""
import ctypes

import numpy as np
import pytest
import torch

import moe_decode_layer_seam_amd as mdl
import synth
from tests import data
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _plan_run(cfg, dinp, dw, m, max_tokens):
    h = mdl.plan(cfg["hidden"], cfg["experts"], cfg["topk"], cfg["inter"], cfg["shared_inter"],
                 max_tokens, cfg["rms_eps"], cfg["routed_scale"], routed=data.routed_of(cfg))
    try:
        out = gu.run(h, cfg, dinp, dw, x=dinp["x"][:m].contiguous()).clone()
        torch.cuda.synchronize()
        assert mdl.status(h) == 0
    finally:
        mdl.destroy(h)
    return out


def _noalloc_run(cfg, dinp, dw, m, max_tokens, status):
    x = dinp["x"][:m].contiguous()
    out = torch.empty_like(x)
    mdl.run_noalloc(cfg, x, dinp["norm_w"], dinp["gate_w"], dinp["bias"], dw["w13"], dw["w13_s"],
                    dw["w2"], dw["w2_s"], dw["sgu"], dw["sgu_s"], dw["sw2"], dw["sw2_s"], out, status,
                    max_tokens=max_tokens, rms_eps=cfg["rms_eps"], routed_scale=cfg["routed_scale"])
    return out


@pytest.mark.parametrize("cfg", [
    dict(synth.WORKLOADS[3], name="dsv41_m48"),
    dict(synth.WORKLOADS[3], routed="mxfp4", name="dsv41_m48_fp4"),
    dict(name="small", m=16, hidden=640, experts=100, topk=8, inter=256, shared_inter=128,
         rms_eps=1e-6, routed_scale=1.0),
], ids=lambda c: c["name"])
def test_noalloc_matches_the_planned_run_on_two_calls(cfg):
    m = cfg["m"]
    inp, w = data.build_layer(17, cfg, experts="picked")
    dinp, dw = gu.inputs_dev(inp), gu.weights_dev(w)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for mm in (m, 3):        # a full step, then a smaller one that routes inside w13
        want = _plan_run(cfg, dinp, dw, mm, m)
        got = _noalloc_run(cfg, dinp, dw, mm, m, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, f"status {int(status.item())} after {mm} rows"
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{mm} rows"


def test_noalloc_rejects_what_it_cannot_hold():
    # 48 rows at hidden 16384 with one expert of I = Is = 8192: the split-mode
    # w2 sums alone need 16 planes x 96 rows x 16384 fp32 = 100 MB, beyond the
    # array.  Every buffer has its real size, so the call is safe whatever it
    # decides.
    H, I, m = 16384, 8192, 48
    cfg = dict(hidden=H, experts=1, topk=1, inter=I, shared_inter=I)
    dev = "cuda"
    x = torch.zeros((m, H), dtype=torch.bfloat16, device=dev)
    t = {
        "norm_w": torch.ones(H, dtype=torch.bfloat16, device=dev),
        "gate_w": torch.zeros((1, H), dtype=torch.bfloat16, device=dev),
        "bias": torch.zeros(1, dtype=torch.float32, device=dev),
        "w13": torch.zeros((1, 2 * I, H), dtype=torch.uint8, device=dev),
        "w13_s": torch.zeros((1, 2 * I // 32, H // 32), dtype=torch.uint8, device=dev),
        "w2": torch.zeros((1, H, I), dtype=torch.uint8, device=dev),
        "w2_s": torch.zeros((1, H // 32, I // 32), dtype=torch.uint8, device=dev),
        "sgu": torch.zeros((2 * I, H), dtype=torch.uint8, device=dev),
        "sgu_s": torch.zeros((2 * I // 32, H // 32), dtype=torch.uint8, device=dev),
        "sw2": torch.zeros((H, I), dtype=torch.uint8, device=dev),
        "sw2_s": torch.zeros((H // 32, I // 32), dtype=torch.uint8, device=dev),
    }
    out = torch.empty_like(x)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(mdl.MoeDecodeError) as err:
        mdl.run_noalloc(cfg, x, t["norm_w"], t["gate_w"], t["bias"], t["w13"], t["w13_s"], t["w2"],
                        t["w2_s"], t["sgu"], t["sgu_s"], t["sw2"], t["sw2_s"], out, status, max_tokens=m)
    assert err.value.code == mdl.EINVAL and "exceeds" in str(err.value)
    # the argument checks of a run: m beyond max_tokens, a null status word
    d = mdl.Dims(H, 1, 1, I, I, 4, 1e-6, 1.0, 0, 0)
    p = [x.data_ptr(), t["norm_w"].data_ptr(), t["gate_w"].data_ptr(), t["bias"].data_ptr()] + \
        [t[n].data_ptr() for n in gu.WEIGHT_NAMES] + [out.data_ptr()]
    assert mdl.lib().moe_decode_run_noalloc(ctypes.byref(d), 5, *p, status.data_ptr(), None) == mdl.EINVAL
    assert mdl.lib().moe_decode_run_noalloc(ctypes.byref(d), 4, *p, None, None) == mdl.EINVAL
    torch.cuda.synchronize()
    assert int(status.item()) == 0
