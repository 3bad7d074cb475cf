"""Pins of the oracle's expert halves and of the rounding-ambiguity rule the
GPU parity tests apply to the SiLU*up intermediate (tests/a8_check.py).

The halves are the expert of the oracle cut in two (page "vllm.models.
deepseek_v41.amd.mono.runner", MonoLayerWeights: w13 gate/up, then w2): the
up half with its sums of magnitudes, and the down half on a given MXFP8
intermediate; the combine is the layer's last step (page "vllm.models.
deepseek_v41.amd.mono.layer", run_ffn).  They are checked against the whole expert and against an
independent torch pipeline (tests/torch_ref.py) on a tiny expert; the
ambiguity rule against values placed exactly on and beside E4M3 rounding
midpoints and E8M0 code boundaries."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import a8_check
from tests import torch_ref as tr


def _expert(seed, H=256, I=128, fmt="e4m3"):
    x = synth.to_bf16_bits(synth.normal(seed, 1, (1, H)))
    y = oracle.rmsnorm(x, synth.to_bf16_bits(synth.normal(seed, 2, (H,), 1.0, 0.1)), 1e-6)
    x8, x8s = oracle.mx_quant_row((np.asarray(y[0], np.uint32) << 16).view(np.float32).astype(np.float64))
    q = oracle.quant_weight_fp4 if fmt == "mxfp4" else oracle.quant_weight
    w13, w13s = q(synth.expert_f32(seed, "w13", 0, 2 * I, H))
    w2, w2s = q(synth.expert_f32(seed, "w2", 0, H, I))
    return x8, x8s, w13, w13s, w2, w2s


@pytest.mark.parametrize("fmt", ["e4m3", "mxfp4"])
def test_halves_make_the_expert(fmt):
    x8, x8s, w13, w13s, w2, w2s = _expert(3, fmt=fmt)
    whole = oracle.expert(x8, x8s, w13, w13s, w2, w2s, fmt=fmt)
    up = oracle.expert_up(x8, x8s, w13, w13s, fmt)
    assert np.array_equal(up["a8"], whole["a8"]) and np.array_equal(up["a8s"], whole["a8s"])
    assert np.array_equal(oracle.expert_down(up["a8"], up["a8s"], w2, w2s, fmt), whole["y"])
    # against torch: h, the sums of magnitudes, and y
    xd = tr.mx_dequant(torch.from_numpy(x8), torch.from_numpy(x8s))
    W13 = tr.dequant(w13, w13s, fmt)
    assert np.allclose(up["h"], (W13 @ xd).numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(up["habs"], (W13.abs() @ xd.abs()).numpy(), rtol=1e-12, atol=0)
    # the down half on another intermediate: torch's dequantised product
    a8 = np.roll(up["a8"], 5)
    W2 = tr.dequant(w2, w2s, fmt)
    want = (W2 @ tr.mx_dequant(torch.from_numpy(a8), torch.from_numpy(up["a8s"]))).numpy()
    assert np.allclose(oracle.expert_down(a8, up["a8s"], w2, w2s, fmt), want, rtol=1e-12, atol=1e-12)


def _up_of(a, h_scale=1.0):
    """A hand-made up half: gate g chosen with SiLU(g) = 1 exactly is not
    possible, so a is given directly with tiny sums (no ambiguity from h)
    and its MXFP8 from the oracle's quantiser."""
    I = a.size
    q, c = oracle.mx_quant_row(a)
    return {"h": np.zeros(2 * I), "habs": np.zeros(2 * I), "a": a, "a8": q, "a8s": c}


def test_ambiguity_is_empty_away_from_midpoints():
    a = np.array([1.0, 1.125, -2.5, 0.75] * 8)         # E4M3 values at code 127... scaled exactly
    up = _up_of(a)
    amb = a8_check.ambiguity(up)
    assert not amb["delta"].any()
    a8_check.check_row(amb, up["a8"], up["a8s"])
    bad = up["a8"].copy()
    bad[3] ^= 1                                        # a neighbouring byte: not allowed here
    with pytest.raises(AssertionError):
        a8_check.check_row(amb, bad, up["a8s"])


def test_ambiguity_allows_both_sides_of_a_midpoint():
    # a group whose largest value sets code 127 (amax 448 scaled: a = 448 *
    # 2^-8 = 1.75), and an element within the arithmetic's error of the
    # midpoint 1.0625 between E4M3 values 1.0 and 1.125 (scaled 2^8 x)
    a = np.full(32, 0.5)
    a[0] = 1.75
    a[5] = 1.0625 / 256 * 256 * (1 + 2.0 ** -30)
    up = _up_of(a)
    up["habs"] = np.full(64, 1.0)                      # error window C_MFMA * 1 on g and u
    up["h"] = np.concatenate([np.full(32, 2.0), np.full(32, 1.0)])
    amb = a8_check.ambiguity(up)
    assert amb["delta"][5] > 0
    other = up["a8"].copy()
    other[5] = oracle.e4m3_rne(1.0 * 2.0 ** (127 - int(up["a8s"][0])))
    assert other[5] != up["a8"][5]
    a8_check.check_row(amb, other, up["a8s"])           # the other rounding is allowed
    far = up["a8"].copy()
    far[5] = oracle.e4m3_rne(1.25 * 2.0 ** (127 - int(up["a8s"][0])))
    with pytest.raises(AssertionError):
        a8_check.check_row(amb, far, up["a8s"])         # two steps away is not


def test_ambiguity_allows_a_code_boundary():
    # amax exactly at 448 * 2^(c - 127) plus a hair: the code may be c or c + 1
    a = np.linspace(-1.0, 1.0, 32)
    a[7] = 448.0 * 2.0 ** -8 * (1 + 2.0 ** -40)
    up = _up_of(a)
    up["habs"] = np.full(64, 1.0)
    up["h"] = np.concatenate([np.full(32, 2.0), np.full(32, 1.0)])
    amb = a8_check.ambiguity(up)
    assert amb["c_hi"][0] == amb["c_lo"][0] + 1
    q2, c2 = oracle.mx_quant_row(a * (1 - 2.0 ** -30))  # the other side of the boundary
    assert c2[0] == amb["c_lo"][0] and up["a8s"][0] == amb["c_hi"][0]
    a8_check.check_row(amb, q2, c2)
    with pytest.raises(AssertionError):
        a8_check.check_row(amb, q2, c2 + 2)


def test_combine_is_the_weighted_sum_then_the_shared_expert():
    # exact binary fractions: the sum is exact, so any order or grouping
    # slip would still pass -- the order is pinned by the cancellation below
    y = np.array([[1.0, 2.0, -0.5], [0.25, -1.0, 4.0]])
    ys = np.array([0.125, 0.0, -3.5])
    out = oracle.combine([0.5, 2.0], y, ys)
    assert np.array_equal(out, 0.5 * y[0] + 2.0 * y[1] + ys)
    # order: w0 y0 + w1 y1 first, then the shared row, in double: 1e16 + 1
    # - 1e16 gives 0 in that order, 1 if the shared row came first
    out = oracle.combine([1.0, 1.0], np.array([[1e16], [1.0]]), np.array([-1e16]))
    assert out[0] == 0.0
