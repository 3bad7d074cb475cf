"""Parity with the oracle over a seeded sweep of shapes, through the C ABI.

The hand-picked cases of test_gpu_parity.py cover the known edges one at a
time; this sweep draws shapes across the whole range the plan accepts (step
widths, hidden and intermediate widths, expert counts, top-k, both routed
formats, the three schedules, and plans made for a wider step than they
run), plus the extremes: one 128-column K step, a single expert, k = 1 and
k = E.  Each case is held to the same bars as the small parity cases
(_check_layer).  The shapes are drawn once, from a fixed seed, so a failing
case keeps its name.
"""
import numpy as np
import pytest
import torch

from tests import data
from tests import gpu_util as gu
from tests.test_gpu_parity import _cfg, _check_layer, _plan_for

pytestmark = pytest.mark.gpu

import moe_decode_layer_seam_amd as mdl  # noqa: E402


def _draw(n, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        m = int(rng.integers(1, 49))
        H = 128 * int(rng.integers(1, 9))
        E = int(rng.integers(1, 301))
        K = int(rng.integers(1, min(E, 32) + 1))
        I = 128 * int(rng.integers(1, 5))
        Is = 128 * int(rng.integers(1, 5))
        c = _cfg(m, H, E, K, I, Is, routed_scale=float(np.round(rng.uniform(0.5, 3.0), 3)))
        c["routed"] = "mxfp4" if i % 3 == 2 else "e4m3"
        c["schedule"] = ("auto", "launches", "persistent")[i % 3]
        c["max_tokens"] = int(rng.integers(m, 49))
        c["name"] = f"s{i}_{c['name']}_{c['routed']}_{c['schedule']}_mx{c['max_tokens']}"
        out.append(c)
    return out


EDGES = [
    dict(_cfg(1, 128, 1, 1, 128, 128), name="edge_one_step_one_expert", max_tokens=1),
    dict(_cfg(48, 128, 1, 1, 128, 128), name="edge_48_rows_one_expert", max_tokens=48),
    dict(_cfg(3, 128, 32, 32, 128, 128), name="edge_k_equals_e", max_tokens=3),
    dict(_cfg(48, 128, 32, 32, 256, 128), name="edge_48_rows_k_equals_e", max_tokens=48),
    dict(_cfg(2, 128, 64, 1, 128, 384, routed="mxfp4"), name="edge_one_step_fp4", max_tokens=7),
]
SWEEP = EDGES + _draw(16)


@pytest.mark.parametrize("cfg", SWEEP, ids=lambda c: c["name"])
def test_parity_sweep(cfg):
    print(f"[sweep] {cfg['name']}", flush=True)
    inp, w = data.build_layer(11, cfg)
    dinp, dw = gu.inputs_dev(inp), gu.weights_dev(w)
    h = _plan_for(cfg, max_tokens=cfg["max_tokens"])
    try:
        out = gu.run(h, cfg, dinp, dw)
        torch.cuda.synchronize()
        _check_layer(cfg, h, inp, w, out)
    finally:
        mdl.destroy(h)
