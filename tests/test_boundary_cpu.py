"""The C ABI library loads on a machine without a GPU, exports every symbol
its header declares, and rejects invalid plans before touching the GPU."""
import ctypes
import os
import re

import pytest

import moe_decode_layer_seam_amd as mdl

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "moe_decode.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_decode_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 10, names
    L = mdl.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(mdl.EXPORTS)


@pytest.mark.parametrize("bad", [
    dict(hidden=100), dict(hidden=0), dict(hidden=32768), dict(experts=0), dict(experts=2048),
    dict(topk=0), dict(topk=9, experts=8), dict(topk=33, experts=64), dict(inter=96),
    dict(shared_inter=0), dict(max_tokens=0), dict(max_tokens=49), dict(rms_eps=-1.0),
    dict(rms_eps=float("nan")), dict(routed_scale=float("inf")), dict(routed_format=2),
    dict(routed_format=-1), dict(schedule=3), dict(schedule=-1),
])
def test_plan_rejects_invalid_dims(bad):
    d = dict(hidden=256, experts=8, topk=2, inter=128, shared_inter=128, max_tokens=4,
             rms_eps=1e-6, routed_scale=1.0, routed_format=0, schedule=0)
    d.update(bad)
    dims = mdl.Dims(d["hidden"], d["experts"], d["topk"], d["inter"], d["shared_inter"],
                    d["max_tokens"], d["rms_eps"], d["routed_scale"], d["routed_format"],
                    d["schedule"])
    h = ctypes.c_void_p()
    assert mdl.lib().moe_decode_plan(ctypes.byref(dims), None, ctypes.byref(h)) == mdl.EINVAL
    assert h.value is None


def test_null_handles_are_rejected():
    L = mdl.lib()
    assert mdl.run_ptrs(None, 1, [0] * 13, stream=0) == mdl.EINVAL
    p, n = ctypes.c_void_p(), ctypes.c_size_t()
    assert L.moe_decode_inspect(None, 0, ctypes.byref(p), ctypes.byref(n)) == mdl.EINVAL
    assert L.moe_decode_timing(None, 1) == mdl.EINVAL
    assert L.moe_decode_quantize_weight(None, 1, 32, 32, None, None, None) == mdl.EINVAL
    assert L.moe_decode_quantize_weight_fp4(None, 1, 32, 32, None, None, None) == mdl.EINVAL
    assert L.moe_decode_quantize_weight_fp4(None, 1, 24, 32, None, None, None) == mdl.EINVAL  # rows % 16
    L.moe_decode_destroy(None)
    assert mdl.strerror(mdl.ECAPTURE) == "called during stream capture"


def test_seam_entry_points_reject_bad_arguments_without_a_gpu():
    L = mdl.lib()
    ok = ctypes.c_void_p(256)  # aligned, never dereferenced: argument checks come first
    args7 = [ok] * 7
    assert L.moe_decode_hc_fold(0, 256, *args7, None) == mdl.EINVAL      # m
    assert L.moe_decode_hc_fold(49, 256, *args7, None) == mdl.EINVAL
    assert L.moe_decode_hc_fold(1, 200, *args7, None) == mdl.EINVAL      # hidden % 128
    assert L.moe_decode_hc_fold(1, 256, *([None] + [ok] * 6), None) == mdl.EINVAL
    # x overlapping the residual
    assert L.moe_decode_hc_fold(1, 256, ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20), ok, ok, ok,
                                ctypes.c_void_p(3 << 20), ctypes.c_void_p((2 << 20) + 512), None) == mdl.EINVAL
    # partial overlap of residual_out and residual
    assert L.moe_decode_hc_fold(1, 256, ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20), ok, ok, ok,
                                ctypes.c_void_p((2 << 20) + 256), ctypes.c_void_p(4 << 20), None) == mdl.EINVAL
    assert L.moe_decode_attn_x8(0, 256, ok, ok, ctypes.c_float(1e-6), ok, ok, None) == mdl.EINVAL
    assert L.moe_decode_attn_x8(1, 96, ok, ok, ctypes.c_float(1e-6), ok, ok, None) == mdl.EINVAL
    assert L.moe_decode_attn_x8(1, 256, ok, ok, ctypes.c_float(-1.0), ok, ok, None) == mdl.EINVAL
    assert L.moe_decode_attn_x8(1, 256, ok, None, ctypes.c_float(1e-6), ok, ok, None) == mdl.EINVAL



def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with a message, before
    touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


# ---- the near-tie rule of the parity tests (host logic) ------------------

def test_near_tie_rule_accepts_ties_and_rejects_real_differences():
    import numpy as np
    from tests import routing_check as rc

    # scores chosen through the logits: b = sigmoid(l) + bias
    E, k = 8, 3
    bias = np.zeros(E)
    logits = np.array([[3.0, 2.0, 1.0, 0.5, 0.0, -1.0, -2.0, -3.0]])
    ref = np.array([[0, 1, 2]])
    assert rc.check_picks(ref, ref, logits, bias) == []
    # a real difference: expert 3 instead of 2 (b lower by ~0.09)
    with pytest.raises(AssertionError):
        rc.check_picks(np.array([[0, 1, 3]]), ref, logits, bias)
    # the order of picks matters beyond the margin
    with pytest.raises(AssertionError):
        rc.check_picks(np.array([[1, 0, 2]]), ref, logits, bias)
    # a boundary near-tie: experts 2 and 3 within 1e-9 of each other
    bias2 = bias.copy()
    s = 1.0 / (1.0 + np.exp(-logits[0]))
    bias2[3] = s[2] - s[3] - 1e-9
    assert rc.check_picks(np.array([[0, 1, 3]]), ref, logits, bias2) == [0]
    # a near-tie between two picks: their order may swap
    bias3 = bias.copy()
    bias3[1] = s[0] - s[1] - 1e-10
    assert rc.check_picks(np.array([[1, 0, 2]]), np.array([[0, 1, 2]]), logits, bias3) == [0]
    # repeated or out-of-range picks never pass
    with pytest.raises(AssertionError):
        rc.check_picks(np.array([[0, 0, 1]]), ref, logits, bias2)
    with pytest.raises(AssertionError):
        rc.check_picks(np.array([[0, 1, 8]]), ref, logits, bias2)
    # weights of given picks: renormalised sigmoid scores
    w = rc.weights_of(np.array([[0, 1, 3]]), logits, 2.0)
    assert np.allclose(w.sum(), 2.0) and np.allclose(w[0, 0] / w[0, 1], s[0] / s[1])
