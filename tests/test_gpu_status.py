"""The status word's failure path, forced from the host.

The launches that route inside w13 (and the persistent launch) wait on other
blocks of the same launch: for the router's logits, for the picks and, in
the persistent launch, at the barriers of an XCD's blocks between its w13,
SiLU * up and w2 phases.  Each wait is bounded; one that runs
past its bound sets a bit of the plan's sticky status word and the wave goes
on, so the run's output is not valid but nothing hangs.  A plan made while
MOE_DECODE_WAIT_LIMIT_US is 0 has every such wait give up at its first
unanswered poll, which happens within a few steps of one token.  The waves
that give up fall back to the shared expert's slots alone, so the run stays
in bounds; the test only checks that the status word reports it, that a
read clears it, and that a plan made without the variable runs clean.
"""
import os
import sys

import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import moe_decode_layer_seam_amd as mdl  # noqa: E402
from tests import data  # noqa: E402
from tests import gpu_util as gu  # noqa: E402

pytestmark = pytest.mark.gpu

# one token, H = 256: routed inside the w13 launch; I = Is = 2048 lets a plan
# of the persistent schedule run the persistent launch
CFG = dict(name="status_m1", m=1, hidden=256, experts=64, topk=6, inter=2048, shared_inter=2048,
           rms_eps=1e-6, routed_scale=1.0)
ROUTE_WAIT, XCD_BARRIER = 2, 1


def _plan(schedule):
    c = CFG
    return mdl.plan(c["hidden"], c["experts"], c["topk"], c["inter"], c["shared_inter"], c["m"],
                    c["rms_eps"], c["routed_scale"], schedule=schedule)


@pytest.mark.parametrize("schedule", ["launches", "persistent"])
def test_waits_that_give_up_set_the_status_word(schedule):
    inp, w = data.build_layer(3, CFG)
    dinp, dw = gu.inputs_dev(inp), gu.weights_dev(w)
    old = os.environ.get("MOE_DECODE_WAIT_LIMIT_US")
    os.environ["MOE_DECODE_WAIT_LIMIT_US"] = "0"
    try:
        h = _plan(schedule)
    finally:
        if old is None:
            del os.environ["MOE_DECODE_WAIT_LIMIT_US"]
        else:
            os.environ["MOE_DECODE_WAIT_LIMIT_US"] = old
    try:
        for _ in range(20):
            gu.run(h, CFG, dinp, dw)
        torch.cuda.synchronize()
        st = mdl.status(h)
        assert st & ROUTE_WAIT, f"no wait for the logits or the picks gave up (status {st})"
        assert st & ~(ROUTE_WAIT | XCD_BARRIER) == 0, f"unexpected status bits {st}"
        assert mdl.status(h) == 0, "reading the status word did not clear it"
    finally:
        mdl.destroy(h)
    # the bound is taken when a plan is made: a plan made now runs clean
    h = _plan(schedule)
    try:
        out = gu.run(h, CFG, dinp, dw)
        torch.cuda.synchronize()
        assert mdl.status(h) == 0
        assert torch.isfinite(out.float()).all()
    finally:
        mdl.destroy(h)
