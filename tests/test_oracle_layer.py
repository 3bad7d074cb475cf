"""Pins of the oracle's layer steps: RMSNorm, router, plan, experts, combine.

Each test checks the oracle against something it does not share code with:
torch library routines (rms_norm, topk, sigmoid, fp8 casts, float64 matmul),
closed forms (the all-zero token), exact invariants (power-of-two scalings,
identical experts, the transpose of a block quantiser) and brute force on
tiny shapes (tests/torch_ref.py).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import data, torch_ref

F64 = torch.float64


def _small_cfg(**kw):
    cfg = dict(name="small", m=5, hidden=256, experts=64, topk=6, inter=128,
               shared_inter=128, rms_eps=1e-6, routed_scale=1.0)
    cfg.update(kw)
    return cfg


# ------------------------------------------------------------- RMSNorm ----

def test_rmsnorm_within_one_bf16_step_of_torch_rms_norm():
    inp = synth.small_inputs(11, 7, 512, 8)
    y = oracle.rmsnorm(inp["x"], inp["norm_w"], 1e-6)
    x = torch_ref.bf16_bits_to_f64(inp["x"])
    w = torch_ref.bf16_bits_to_f64(inp["norm_w"])
    ref = torch.nn.functional.rms_norm(x, (512,), w, eps=1e-6).numpy()
    got = torch_ref.bf16_bits_to_f64(y).numpy()
    # three roundings (fp32, fp32, bf16): within 2^-8 relative of the exact norm
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)


def test_rmsnorm_power_of_two_scaling_is_exact():
    # With eps = 0, scaling a row by 2^k scales ss/H by 4^k and r by 2^-k
    # exactly, so the normed row is unchanged bit for bit.
    inp = synth.small_inputs(12, 4, 256, 8)
    x = inp["x"].astype(np.uint32)
    x4 = (x + (2 << 7)).astype(np.uint16)  # +2 on the bf16 exponent: * 4
    nz = (x & 0x7FFF) != 0
    x4 = np.where(nz, x4, inp["x"])
    y1 = oracle.rmsnorm(inp["x"], inp["norm_w"], 0.0)
    y2 = oracle.rmsnorm(x4, inp["norm_w"], 0.0)
    assert np.array_equal(y1, y2)


def test_rmsnorm_zero_row_is_positive_zero():
    inp = synth.small_inputs(13, 2, 256, 8)
    x = np.zeros((2, 256), np.uint16)
    y = oracle.rmsnorm(x, inp["norm_w"], 1e-6)  # norm_w ~ 1 + N(0, 0.1) > 0
    assert np.all(y == 0)


# -------------------------------------------------------------- Router ----

def test_router_without_bias_is_torch_topk_of_logits():
    inp = synth.small_inputs(21, 9, 256, 64)
    y = oracle.rmsnorm(inp["x"], inp["norm_w"], 1e-6)
    r = oracle.router(y, inp["gate_w"], np.zeros(64, np.float32), 8)
    lg = torch_ref.bf16_bits_to_f64(y) @ torch_ref.bf16_bits_to_f64(inp["gate_w"]).T
    assert np.allclose(r["logits"], lg.numpy(), rtol=1e-13, atol=1e-13)
    top = torch.topk(lg, 8, dim=-1)  # sigmoid is monotone: same order
    assert np.array_equal(r["ids"], top.indices.numpy())
    s = torch.sigmoid(top.values)
    assert np.allclose(r["wts"], (s / s.sum(-1, keepdim=True)).numpy(), rtol=1e-14)


def test_router_ties_go_to_the_lower_expert():
    inp = synth.small_inputs(22, 1, 256, 8)
    g = inp["gate_w"].copy()
    g[5] = g[3]           # experts 3 and 5 now score identically
    bias = np.full(8, -1.0, np.float32)
    bias[3] = bias[5] = 1.0
    y = oracle.rmsnorm(inp["x"], inp["norm_w"], 1e-6)
    assert list(oracle.router(y, g, bias, 1)["ids"][0]) == [3]
    r = oracle.router(y, g, bias, 2)
    assert list(r["ids"][0]) == [3, 5] and r["margin"][0] > 0
    assert r["wts"][0, 0] == r["wts"][0, 1] == 0.5


def test_router_k_equals_e_weights_are_normalised_scores():
    inp = synth.small_inputs(23, 3, 256, 8)
    y = oracle.rmsnorm(inp["x"], inp["norm_w"], 1e-6)
    r = oracle.router(y, inp["gate_w"], inp["bias"], 8, routed_scale=2.5)
    s = torch.sigmoid(torch.from_numpy(r["logits"]))
    want = 2.5 * s / s.sum(-1, keepdim=True)
    got = np.zeros((3, 8))
    np.put_along_axis(got, r["ids"].astype(np.int64), r["wts"], axis=1)
    assert np.allclose(got, want.numpy(), rtol=1e-14)
    b = s.numpy() + inp["bias"].astype(np.float64)
    assert np.array_equal(r["ids"], np.argsort(-b, axis=1, kind="stable"))


# ---------------------------------------------------------------- Plan ----

def test_plan_invariants():
    rng = np.random.default_rng(31)
    m, E, k = 37, 50, 6
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(m)]).astype(np.int32)
    counts, row = oracle.plan(ids, E)
    assert counts.sum() == m * k
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    assert np.array_equal(np.sort(row.ravel()), np.arange(m * k))  # each pair once
    # rows listed by expert ascending, then token ascending
    order = np.argsort(row.ravel())
    e_of = ids.ravel()[order]
    t_of = order // k
    key = e_of.astype(np.int64) * m + t_of
    assert np.all(np.diff(key) > 0)


# ------------------------------------------------------------- Experts ----

def test_expert_matches_torch_reference():
    cfg = _small_cfg()
    inp, w = data.build_layer(41, cfg, experts=[0, 7, 63])
    y = oracle.rmsnorm(inp["x"], inp["norm_w"], 1e-6)
    xq, xc = torch_ref.mx_quant(torch_ref.bf16_bits_to_f64(y))
    for t in range(cfg["m"]):
        for e in (0, 7, 63):
            o = oracle.expert(xq[t].numpy(), xc[t].numpy(), w["w13"][e], w["w13_s"][e],
                              w["w2"][e], w["w2_s"][e])
            ry, ra, rc = torch_ref.expert(xq[t], xc[t], w["w13"][e], w["w13_s"][e],
                                          w["w2"][e], w["w2_s"][e])
            assert np.array_equal(o["a8"], ra.numpy()) and np.array_equal(o["a8s"], rc.numpy())
            assert np.allclose(o["y"], ry.numpy(), rtol=1e-12, atol=1e-15)


def test_expert_gemm_exact_for_unit_scales():
    # All codes 127 and small-integer E4M3 values: every product and partial
    # sum of the first GEMM is an integer below 2^53, so h equals numpy's
    # integer matmul exactly, and with it the quantised intermediate.
    rng = np.random.default_rng(42)
    H, I = 256, 64
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0xC4])  # 0, 1,2,3,4, -1,-2,-3
    vals = np.array([0, 1, 2, 3, 4, -1, -2, -3], np.int64)
    xi = rng.integers(0, 8, H)
    wi = rng.integers(0, 8, (2 * I, H))
    w2i = rng.integers(0, 8, (H, I))
    x8 = ints[xi].astype(np.uint8)
    w13 = ints[wi].astype(np.uint8)
    w2 = ints[w2i].astype(np.uint8)
    ones = lambda r, c: np.full((r, c), 127, np.uint8)
    o = oracle.expert(x8, np.full(H // 32, 127, np.uint8), w13, ones(2 * I // 32, H // 32),
                      w2, ones(H // 32, I // 32))
    h = vals[wi] @ vals[xi]
    g, u = h[:I].astype(np.float64), h[I:].astype(np.float64)
    a = torch.from_numpy(g * (1 / (1 + np.exp(-g))) * u).to(torch.float32).to(F64)
    aq, ac = torch_ref.mx_quant(a)
    assert np.array_equal(o["a8"], aq.numpy()) and np.array_equal(o["a8s"], ac.numpy())
    yref = vals[w2i].astype(np.float64) @ torch_ref.mx_dequant(aq, ac).numpy()
    assert np.allclose(o["y"], yref, rtol=1e-14, atol=0)


def test_expert_w2_scale_plus_one_doubles_exactly():
    cfg = _small_cfg()
    inp, w = data.build_layer(43, cfg, experts=[5])
    y = oracle.rmsnorm(inp["x"], inp["norm_w"], 1e-6)
    xq, xc = torch_ref.mx_quant(torch_ref.bf16_bits_to_f64(y))
    a = oracle.expert(xq[0].numpy(), xc[0].numpy(), w["w13"][5], w["w13_s"][5], w["w2"][5], w["w2_s"][5])
    b = oracle.expert(xq[0].numpy(), xc[0].numpy(), w["w13"][5], w["w13_s"][5], w["w2"][5],
                      (w["w2_s"][5] + 1).astype(np.uint8))
    assert np.array_equal(b["y"], 2 * a["y"])


# ----------------------------------------------------- Weight quantiser ----

def test_weight_quantiser_transpose_equivariant():
    w = synth.normal(44, 99, (96, 160), 0.0, 0.02)
    q, s = oracle.quant_weight(w)
    qt, st = oracle.quant_weight(np.ascontiguousarray(w.T))
    assert np.array_equal(q.T, qt) and np.array_equal(s.T, st)


def test_weight_quantiser_block_layout_and_error_bound():
    w = synth.normal(45, 98, (64, 128), 0.0, 0.02)
    w[33, 70] = 5.0   # block (1, 2) gets a large amax
    q, s = oracle.quant_weight(w)
    assert s.shape == (2, 4)
    big = oracle.mx_code(5.0)
    assert s[1, 2] == big and np.all(np.delete(s.ravel(), 1 * 4 + 2) < big)
    dq = torch_ref.block_dequant(q, s).numpy()
    scaled = np.abs(w.astype(np.float64)) * np.exp2(127.0 - np.repeat(np.repeat(s, 32, 0), 32, 1))
    normal = scaled >= 2.0 ** -6
    assert np.all(np.abs(dq - w)[normal] <= 2.0 ** -4 * np.abs(w)[normal])


# ------------------------------------------------------- Whole layer ----

@pytest.mark.parametrize("cfg", [synth.WORKLOADS[0], _small_cfg(),
                                 _small_cfg(m=3, experts=8, topk=8, routed_scale=2.5)])
def test_layer_matches_torch_reference_on_tiny_shapes(cfg):
    inp, w = data.build_layer(51, cfg)
    o = oracle.layer(data.dims_of(cfg), inp, w)
    r = torch_ref.layer(data.dims_of(cfg), inp, w, o["normed"])
    assert np.array_equal(o["x8"], r["x8"]) and np.array_equal(o["x8s"], r["x8s"])
    assert np.array_equal(o["ids"], r["ids"])
    assert np.allclose(o["wts"], r["wts"], rtol=1e-14)
    assert np.allclose(o["out_f64"], r["out_f64"], rtol=1e-11, atol=1e-14)
    ref_bits = oracle.bf16_rne_array(o["out_f64"]).reshape(o["out"].shape)
    assert np.array_equal(o["out"], ref_bits)


def test_layer_zero_token_closed_form():
    cfg = _small_cfg(m=2)
    inp, w = data.build_layer(52, cfg)
    inp = dict(inp, x=np.zeros_like(inp["x"]))
    o = oracle.layer(data.dims_of(cfg), inp, w)
    assert np.all(o["normed"] == 0) and np.all(o["x8"] == 0) and np.all(o["x8s"] == 0)
    assert np.all(o["logits"] == 0)
    # sigmoid(0) = 1/2 for every expert: the picks are the top-k of the bias
    want = np.argsort(-inp["bias"].astype(np.float64), kind="stable")[:cfg["topk"]]
    assert np.all(o["ids"] == want[None, :])
    assert np.all(o["wts"] == 1.0 / cfg["topk"])
    assert np.all(o["out"] == 0) and np.all(o["out_f64"] == 0)


def test_layer_identical_experts_make_routing_irrelevant():
    cfg = _small_cfg(m=3, experts=16, topk=4, routed_scale=1.5)
    inp, w = data.build_layer(53, cfg, experts=[0])
    for n in ("w13", "w13_s", "w2", "w2_s"):
        w[n][:] = w[n][0]
    o1 = oracle.layer(data.dims_of(cfg), inp, w)
    inp2 = dict(inp, bias=synth.normal(99, 4, (16,), 0.0, 1.0))
    o2 = oracle.layer(data.dims_of(cfg), inp2, w)
    assert not np.array_equal(o1["ids"], o2["ids"])
    assert np.allclose(o1["out_f64"], o2["out_f64"], rtol=1e-13, atol=1e-15)
    for t in range(3):
        e = oracle.expert(o1["x8"][t], o1["x8s"][t], w["w13"][0], w["w13_s"][0], w["w2"][0], w["w2_s"][0])
        s = oracle.expert(o1["x8"][t], o1["x8s"][t], w["sgu"], w["sgu_s"], w["sw2"], w["sw2_s"])
        assert np.allclose(o1["out_f64"][t], 1.5 * e["y"] + s["y"], rtol=1e-13, atol=1e-15)
