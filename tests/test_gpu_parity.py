"""Parity of the HIP path with the oracle, through the C ABI.

Bars: bit-exact for the normed bf16 rows, the MXFP8 activation bytes and
codes, the picked experts and the plan (up to near-ties of the biased score,
tests/routing_check.py); routing weights within 1e-6 relative; every byte and
code of the SiLU*up intermediate one of the roundings the arithmetic allows
(tests/a8_check.py); |gpu - ref| <= 1e-2 + 2e-2 |ref| for the bf16 output
(ref: the oracle's double-precision sum before its rounding), plus the part
an allowed different rounding of the intermediate can move each element.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from concurrent.futures import ThreadPoolExecutor

from tests import a8_check
from tests import data
from tests import gpu_util as gu
from tests import routing_check

pytestmark = pytest.mark.gpu

import moe_decode_layer_seam_amd as mdl  # noqa: E402


def _cfg(m, H, E, K, I, Is, **kw):
    c = dict(name=f"m{m}_h{H}_e{E}_k{K}_i{I}_is{Is}", m=m, hidden=H, experts=E, topk=K,
             inter=I, shared_inter=Is, rms_eps=1e-6, routed_scale=1.0)
    c.update(kw)
    if "schedule" in kw:
        c["name"] += "_" + kw["schedule"]
    return c


SMALL = [
    synth.WORKLOADS[0],
    _cfg(1, 256, 64, 6, 128, 128),
    _cfg(5, 512, 64, 6, 256, 128),          # I != Is
    _cfg(13, 640, 100, 8, 128, 256),        # H % 512 != 0, E not a multiple of 64
    _cfg(16, 256, 256, 8, 128, 128),
    _cfg(17, 384, 256, 8, 256, 256, routed_scale=2.5),
    _cfg(33, 256, 8, 8, 128, 128),          # k = E
    _cfg(48, 512, 64, 4, 256, 256),
    _cfg(48, 256, 512, 16, 128, 128),       # 8 sort groups, k = 16
    _cfg(7, 256, 1000, 32, 128, 128),       # 16 sort groups, k = 32
    _cfg(48, 256, 1024, 32, 128, 128),      # the largest plan: 1536 picks over 1024 experts
    _cfg(48, 640, 100, 8, 1024, 512),       # w13 in whole units over a ragged last K segment
    # m <= 4: the seam and router inside the w13 launch (ragged H, E), and the
    # cases that keep their own launches (E > 256, m k > 64, H > 8192)
    _cfg(4, 640, 100, 8, 128, 256),
    _cfg(2, 256, 300, 8, 128, 128),
    _cfg(4, 256, 64, 20, 128, 128),
    _cfg(2, 8320, 16, 2, 128, 128),
    # m <= 4 with I and Is of 2048 or 4096: the persistent launch, cut by XCD
    # (ragged H and E, I != Is, k = 1)
    _cfg(1, 256, 64, 6, 2048, 2048, schedule="persistent"),
    _cfg(4, 640, 100, 8, 2048, 4096, schedule="persistent"),
    _cfg(3, 512, 256, 8, 4096, 2048, schedule="persistent"),
    _cfg(2, 384, 16, 1, 2048, 2048, schedule="persistent"),
]


def _plan_for(cfg, max_tokens=None, schedule=None):
    schedule = schedule or cfg.get("schedule", "auto")
    return mdl.plan(cfg["hidden"], cfg["experts"], cfg["topk"], cfg["inter"],
                    cfg["shared_inter"], max_tokens or cfg["m"], cfg["rms_eps"],
                    cfg["routed_scale"], routed=data.routed_of(cfg), schedule=schedule)


def _check_layer(cfg, handle, inp, w, out, rows_ref=None, o=None):
    """Compare every intermediate of the last run with the oracle."""
    m, H, E, K = cfg["m"], cfg["hidden"], cfg["experts"], cfg["topk"]
    dims = data.dims_of(cfg)
    assert mdl.status(handle) == 0, "a wait inside a launch timed out"
    # norm, quant and router for every row (cheap on the CPU)
    y = oracle.rmsnorm(inp["x"], inp["norm_w"], cfg["rms_eps"])
    assert np.array_equal(gu.tap(handle, "normed", torch.int16).view(np.uint16).reshape(m, H), y)
    x8 = np.empty((m, H), np.uint8)
    x8s = np.empty((m, H // 32), np.uint8)
    for t in range(m):
        x8[t], x8s[t] = oracle.mx_quant_row(_bf16_f64(y[t]))
    assert np.array_equal(gu.tap(handle, "x8").reshape(m, H), x8)
    assert np.array_equal(gu.tap(handle, "x8s").reshape(m, H // 32), x8s)
    r = oracle.router(y, inp["gate_w"], inp["bias"], K, cfg["routed_scale"])
    logits = gu.tap(handle, "logits", torch.float64).reshape(m, E)
    assert np.allclose(logits, r["logits"], rtol=1e-12, atol=1e-12)
    ids = gu.tap(handle, "topk_ids", torch.int32).reshape(m, K)
    # ids bit-exact, except near-ties at the top-k boundary (or between picks)
    # that leave a valid top-k of the oracle's biased scores
    ties = routing_check.check_picks(ids, r["ids"], r["logits"], inp["bias"])
    if ties:
        print(f"[{cfg['name']}] near-tie picks at tokens {ties}; oracle margins "
              f"{r['margin'][ties]}", flush=True)
    assert len(ties) <= max(1, m // 16), f"too many near-ties to be chance: {ties}"
    wts = gu.tap(handle, "topk_w", torch.float32).reshape(m, K)
    want_w = r["wts"].copy()
    if ties:
        want_w[ties] = routing_check.weights_of(ids[ties], r["logits"][ties], cfg["routed_scale"])
    assert np.allclose(wts, want_w, rtol=1e-6, atol=0)
    # the plan of the picks the run made
    counts, row = oracle.plan(ids, E)
    assert np.array_equal(gu.tap(handle, "counts", torch.int32), counts)
    assert np.array_equal(gu.tap(handle, "pair_row", torch.int32).reshape(m, K), row)
    row_tok = gu.tap(handle, "row_tok", torch.int32)
    want_tok = np.empty(m * K + m, np.int32)
    want_tok[row.ravel()] = np.repeat(np.arange(m), K)
    want_tok[m * K:] = np.arange(m)
    assert np.array_equal(row_tok, want_tok)
    # output rows (all, or a sample), less the near-tie tokens: their output
    # follows other picks than the oracle's
    rows = list(range(m)) if rows_ref is None else list(rows_ref)
    if o is None:
        o = oracle.layer_parallel(dims, inp, w, rows, workers=data.WORKERS)
    keep = [i for i, t in enumerate(rows) if t not in ties]
    # the intermediate: every GPU byte must be the oracle's or, where the
    # oracle's value lies within the arithmetic's error of a rounding
    # midpoint, the other correct rounding (tests/a8_check.py); the output is
    # then held to the bar against the oracle's down projection and combine
    # of those bytes.  With no differing byte that reference is the oracle's
    # own output.
    ref, nb, nc = _reference_out(cfg, handle, o, w, [rows[i] for i in keep], keep, ids, row)
    got = gu.out_f64(out)[rows][keep]
    gu.assert_out_close(got, ref, what=cfg["name"])
    plain = np.abs(got - o["out_f64"][keep]) > 1e-2 + 2e-2 * np.abs(o["out_f64"][keep])
    print(f"[{cfg['name']}] intermediate bytes differing from the oracle's: {nb}, codes: {nc}; "
          f"output elements beyond the bar against the oracle's own intermediate: {int(plain.sum())}",
          flush=True)
    return r, o


def _reference_out(cfg, handle, o, w, toks, idx, ids, row):
    """For token rows `toks` (o's rows `idx`): checks every SiLU*up byte and
    code of the GPU run against the roundings the arithmetic allows, then
    returns the oracle's output [len(toks), H] computed from those bytes
    (its down projection of each expert's intermediate and its combine),
    with the counts of bytes and codes that differ from the oracle's."""
    m, H, K = cfg["m"], cfg["hidden"], cfg["topk"]
    I, Is = cfg["inter"], cfg["shared_inter"]
    Imax = max(I, Is)
    fmt = data.routed_of(cfg)
    a8 = gu.tap(handle, "a8").reshape(-1, Imax)
    a8s = gu.tap(handle, "a8s").reshape(-1, Imax // 32)

    def one(job):
        t, i = job
        ys = np.empty((K, H))
        nb = nc = 0
        for j in range(K + 1):
            if j < K:
                e = int(ids[t, j])
                w13, w13s, w2, w2s, f, Kv, gr = (w["w13"][e], w["w13_s"][e], w["w2"][e], w["w2_s"][e],
                                                 fmt, I, int(row[t, j]))
            else:
                w13, w13s, w2, w2s, f, Kv, gr = w["sgu"], w["sgu_s"], w["sw2"], w["sw2_s"], "e4m3", Is, m * K + t
            up = oracle.expert_up(o["x8"][i], o["x8s"][i], w13, w13s, f)
            a8_g, a8s_g = a8[gr, :Kv], a8s[gr, :Kv // 32]
            a8_check.check_row(a8_check.ambiguity(up), a8_g, a8s_g)
            db, dc = a8_check.differing(up, a8_g, a8s_g)
            nb, nc = nb + db, nc + dc
            y = oracle.expert_down(a8_g, a8s_g, w2, w2s, f)
            if j < K:
                ys[j] = y
            else:
                ysh = y
        return oracle.combine(o["wts"][i], ys, ysh), nb, nc

    with ThreadPoolExecutor(max_workers=data.WORKERS) as ex:
        res = list(ex.map(one, list(zip(toks, idx))))
    ref = np.stack([r_[0] for r_ in res]) if res else np.zeros((0, H))
    return ref, sum(r_[1] for r_ in res), sum(r_[2] for r_ in res)


def _bf16_f64(bits):
    """bf16 bit patterns -> their values as float64."""
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


# MXFP4 (E2M1 pairs, 1 x 32 codes) routed experts: odd K step counts (H 640,
# I 128) leave one half of a weight line pair empty
SMALL_FP4 = [dict(c, routed="mxfp4", name=c["name"] + "_fp4") for c in (
    synth.WORKLOADS[0],
    _cfg(4, 640, 100, 8, 128, 256),
    _cfg(5, 512, 64, 6, 256, 128),
    _cfg(13, 640, 100, 8, 128, 256),
    _cfg(33, 256, 8, 8, 128, 128),
    _cfg(48, 512, 64, 4, 256, 256),
    _cfg(7, 256, 1000, 32, 128, 128),
    _cfg(48, 640, 100, 8, 1024, 512),
)]


@pytest.mark.parametrize("cfg", SMALL + SMALL_FP4, ids=lambda c: c["name"])
def test_parity_small(cfg):
    inp, w = data.build_layer(7, cfg)
    dinp, dw = gu.inputs_dev(inp), gu.weights_dev(w)
    h = _plan_for(cfg, max_tokens=48)
    try:
        out = gu.run(h, cfg, dinp, dw)
        torch.cuda.synchronize()
        _check_layer(cfg, h, inp, w, out)
    finally:
        mdl.destroy(h)


def test_parity_with_widely_varying_block_codes():
    """Block codes that differ from block to block by up to +-6 (weights and
    activations), so a scale applied to the wrong 32-column block or the
    wrong row block changes the output far beyond the tolerance."""
    cfg = _cfg(6, 512, 16, 4, 256, 128)
    H, E, I, Is = 512, 16, 256, 128
    inp = synth.small_inputs(21, 6, H, E)
    rng = np.random.default_rng(21)
    # activations: each 32-column group of x scaled by its own power of two
    xf = synth.normal(21, 1, (6, H)) * np.exp2(rng.integers(-6, 7, (6, H // 32))).repeat(32, 1)
    inp["x"] = synth.to_bf16_bits(xf.astype(np.float32))
    w = data.alloc_weights(cfg)

    def q(name, shape):
        f = synth.normal(21, synth.STREAM[name], shape, 0.0, 0.02)
        f = f * np.exp2(rng.integers(-6, 7, (shape[0] // 32, shape[1] // 32))).repeat(32, 0).repeat(32, 1)
        return oracle.quant_weight(f.astype(np.float32))

    for e in range(E):
        w["w13"][e], w["w13_s"][e] = q("w13", (2 * I, H))
        w["w2"][e], w["w2_s"][e] = q("w2", (H, I))
    w["sgu"], w["sgu_s"] = q("sgu", (2 * Is, H))
    w["sw2"], w["sw2_s"] = q("sw2", (H, Is))
    assert len(np.unique(w["w13_s"])) > 8 and len(np.unique(w["sw2_s"])) > 8
    dinp, dw = gu.inputs_dev(inp), gu.weights_dev(w)
    h = _plan_for(cfg)
    try:
        out = gu.run(h, cfg, dinp, dw)
        torch.cuda.synchronize()
        _check_layer(cfg, h, inp, w, out)
    finally:
        mdl.destroy(h)


def test_zero_tokens_give_exact_zero():
    cfg = _cfg(9, 512, 64, 6, 128, 128)
    inp, w = data.build_layer(8, cfg)
    inp["x"] = np.zeros_like(inp["x"])
    dinp, dw = gu.inputs_dev(inp), gu.weights_dev(w)
    h = _plan_for(cfg)
    try:
        out = gu.run(h, cfg, dinp, dw)
        torch.cuda.synchronize()
        assert torch.all(out.view(torch.int16) == 0)
        assert np.all(gu.tap(h, "x8") == 0) and np.all(gu.tap(h, "x8s") == 0)
        want = np.argsort(-inp["bias"].astype(np.float64), kind="stable")[:6]
        ids = gu.tap(h, "topk_ids", torch.int32).reshape(9, 6)
        assert np.all(ids == want[None, :])
    finally:
        mdl.destroy(h)


def test_concentrated_routing_splits_slots():
    # every token picks the same experts: 48 rows per expert, three token tiles
    cfg = _cfg(48, 256, 64, 4, 128, 128)
    inp, w = data.build_layer(9, cfg)
    inp["bias"] = inp["bias"].copy()
    inp["bias"][[3, 17, 40, 63]] = 10.0
    dinp, dw = gu.inputs_dev(inp), gu.weights_dev(w)
    h = _plan_for(cfg)
    try:
        out = gu.run(h, cfg, dinp, dw)
        torch.cuda.synchronize()
        _check_layer(cfg, h, inp, w, out)
    finally:
        mdl.destroy(h)


@pytest.mark.parametrize("schedule,inter", [("launches", 256), ("persistent", 2048)])
def test_runs_are_deterministic_and_plan_reusable_across_m(schedule, inter):
    # persistent at I = 2048: steps of up to 4 rows run the persistent
    # launch, the others the short launches, and a token's bits are the same
    # in either
    cfg = _cfg(48, 512, 256, 8, inter, inter)
    inp, w = data.build_layer(10, cfg)
    dinp, dw = gu.inputs_dev(inp), gu.weights_dev(w)
    h = _plan_for(cfg, schedule=schedule)
    try:
        a = gu.run(h, cfg, dinp, dw).clone()
        b = gu.run(h, cfg, dinp, dw).clone()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        # smaller steps on the same plan (m = 3 computes the router logits in
        # the seam launch, m = 5 and 48 in their own), then the full one again
        c = gu.run(h, cfg, dinp, dw, x=dinp["x"][:5].contiguous()).clone()
        c3 = gu.run(h, cfg, dinp, dw, x=dinp["x"][:3].contiguous()).clone()
        d = gu.run(h, cfg, dinp, dw)
        # steps of up to 4 tokens route inside the w13 launch: twice in a row,
        # after a larger step, and with another token count
        e3 = gu.run(h, cfg, dinp, dw, x=dinp["x"][:3].contiguous()).clone()
        e3b = gu.run(h, cfg, dinp, dw, x=dinp["x"][:3].contiguous()).clone()
        e1 = gu.run(h, cfg, dinp, dw, x=dinp["x"][:1].contiguous()).clone()
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), a[:5].view(torch.int16))
        assert torch.equal(c3.view(torch.int16), a[:3].view(torch.int16))
        assert torch.equal(d.view(torch.int16), a.view(torch.int16))
        assert torch.equal(e3.view(torch.int16), a[:3].view(torch.int16))
        assert torch.equal(e3b.view(torch.int16), a[:3].view(torch.int16))
        assert torch.equal(e1.view(torch.int16), a[:1].view(torch.int16))
        assert mdl.status(h) == 0
    finally:
        mdl.destroy(h)


def test_whole_and_split_units_give_the_same_bits():
    """Batch invariance across the GEMM modes: on the draft layer's shape (H
    5120, 64 experts top-4, I = Is = 1024) 48 rows run w13 and w2 in whole
    units, 8 and 5 rows in split units, and 1 row routes inside the w13
    launch; a token's output bits are the same in each."""
    cfg = dict(synth.WORKLOADS[4], name="draft_modes")
    dw = _gpu_weights(cfg, 41)
    inp = synth.small_inputs(9, 48, cfg["hidden"], cfg["experts"])
    dinp = gu.inputs_dev(inp)
    h = _plan_for(cfg)
    try:
        full = gu.run(h, cfg, dinp, dw).clone()
        parts = {n: gu.run(h, cfg, dinp, dw, x=dinp["x"][:n].contiguous()).clone() for n in (8, 5, 1)}
        torch.cuda.synchronize()
        assert mdl.status(h) == 0
        for n, o in parts.items():
            assert torch.equal(o.view(torch.int16), full[:n].view(torch.int16)), f"{n} rows"
    finally:
        mdl.destroy(h)


# m = 3: the launches schedule runs the seam and the router inside the w13
# launch, whose hand-off boxes the act launch clears for the next replay
@pytest.mark.parametrize("schedule,m,inter", [("launches", 16, 256), ("launches", 3, 256), ("persistent", 3, 2048)])
def test_graph_capture_replays_match_eager(schedule, m, inter):
    # ("auto", 3, 2048): the persistent launch and the combine launch that
    # clears its hand-off words for the next replay
    cfg = _cfg(m, 512, 64, 6, inter, 2048 if inter == 2048 else 128)
    inp, w = data.build_layer(11, cfg)
    dinp, dw = gu.inputs_dev(inp), gu.weights_dev(w)
    h = _plan_for(cfg, schedule=schedule)
    try:
        xs = [gu.bf16_dev(synth.to_bf16_bits(synth.normal(100 + i, 1, (m, 512)))) for i in range(4)]
        eager = []
        for x in xs:
            eager.append(gu.run(h, cfg, dinp, dw, x=x).clone())
        torch.cuda.synchronize()
        xin = torch.empty_like(xs[0])
        out = torch.empty_like(xs[0])
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            gu.run(h, cfg, dinp, dw, x=xin, out=out)  # warm-up outside the graph
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gu.run(h, cfg, dinp, dw, x=xin, out=out)
        for rep in range(3):
            for i, x in enumerate(xs):
                xin.copy_(x)
                g.replay()
                torch.cuda.synchronize()
                assert torch.equal(out.view(torch.int16), eager[i].view(torch.int16)), (rep, i)
        assert mdl.status(h) == 0
        del g
    finally:
        mdl.destroy(h)


def _gpu_weights(cfg, seed):
    """N(0, 0.02) weights drawn on the GPU and quantised by the library."""
    E, H, I, Is = cfg["experts"], cfg["hidden"], cfg["inter"], cfg["shared_inter"]
    fp4 = data.routed_of(cfg) == "mxfp4"
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = {}

    def make(name, shape, routed):
        w = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * 0.02
        rows, cols = shape[-2], shape[-1]
        if routed and fp4:
            q = torch.empty(shape[:-1] + (cols // 2,), dtype=torch.uint8, device="cuda")
            sc = torch.empty(shape[:-2] + mdl.fp4_codes_shape(rows, cols), dtype=torch.uint8, device="cuda")
            mdl.quantize_weight_fp4(w, q, sc)
        else:
            q = torch.empty(shape, dtype=torch.uint8, device="cuda")
            sc = torch.empty(shape[:-2] + (rows // 32, cols // 32), dtype=torch.uint8, device="cuda")
            mdl.quantize_weight(w, q, sc)
        out[name], out[name + "_s"] = q, sc

    make("w13", (E, 2 * I, H), True)
    make("w2", (E, H, I), True)
    make("sgu", (2 * Is, H), False)
    make("sw2", (H, Is), False)
    return out


# steps the persistent launch covers: the full layer at 1, 3 and 4 rows, a
# shape with Is = 4096, and 2 rows at k = 1
PERSISTENT_CASES = [
    dict(synth.WORKLOADS[1], name="dsv41_m1"),
    dict(synth.WORKLOADS[1], m=3, name="dsv41_m3"),
    dict(synth.WORKLOADS[1], m=4, name="dsv41_m4"),
    _cfg(4, 640, 100, 8, 2048, 4096),
    _cfg(2, 384, 16, 1, 2048, 2048),
]


@pytest.mark.parametrize("cfg", PERSISTENT_CASES, ids=lambda c: c["name"])
def test_persistent_launch_matches_the_short_launches_bit_for_bit(cfg):
    """In a plan of the persistent schedule, a step of m <= 4 rows runs the
    persistent launch (its timing event records the dispatches) and a step of
    5 rows the short launches, with the same arithmetic in the same order --
    the w2 segments are the XCD slices -- so the m rows come out the same
    bytes in either."""
    m, H, E = cfg["m"], cfg["hidden"], cfg["experts"]
    dw = _gpu_weights(cfg, 31)
    dinp = gu.inputs_dev(synth.small_inputs(5, 5, H, E))
    h = _plan_for(cfg, max_tokens=5, schedule="persistent")
    try:
        mdl.timing(h, True)
        outs = [gu.run(h, cfg, dinp, dw, x=dinp["x"][:m].contiguous()).clone() for _ in range(2)]
        torch.cuda.synchronize()
        _, runs = mdl.timing_read(h, "persistent")
        assert runs == 2, runs
        five = gu.run(h, cfg, dinp, dw).clone()
        torch.cuda.synchronize()
        _, runs = mdl.timing_read(h, "persistent")
        assert runs == 2, runs  # the 5-row step ran the short launches
        mdl.timing(h, False)
        assert mdl.status(h) == 0
    finally:
        mdl.destroy(h)
    for o in outs:
        assert torch.equal(o.view(torch.int16), five[:m].view(torch.int16))


def test_quantize_weight_matches_oracle():
    w = synth.normal(12, 77, (3, 256, 320), 0.0, 0.02)
    w[0, :32, :32] = 0.0                      # all-zero block: code 0
    w[1, 32:64, 64:96] *= 1e-30               # tiny block
    w[2, 100, 200] = 300.0                    # a spike
    w[2, 5, 7] = -1e-41                       # a subnormal
    q_ref = np.empty(w.shape, np.uint8)
    s_ref = np.empty((3, 8, 10), np.uint8)
    for i in range(3):
        q_ref[i], s_ref[i] = oracle.quant_weight(w[i])
    wd = torch.from_numpy(w).cuda()
    q = torch.empty(w.shape, dtype=torch.uint8, device="cuda")
    s = torch.empty((3, 8, 10), dtype=torch.uint8, device="cuda")
    mdl.quantize_weight(wd, q, s)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_quantize_weight_fp4_matches_oracle():
    w = synth.normal(14, 78, (2, 96, 320), 0.0, 0.02)
    w[0, 0, :32] = 0.0                        # all-zero group: code 0
    w[0, 1, 32:64] *= 1e-30                   # tiny group
    w[1, 5, 100] = 300.0                      # a spike
    w[1, 6, 7] = -1e-41                       # a subnormal
    w[1, 7, 64:96] = np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4)  # ties (code 127)
    # 320 columns: one ragged 512-column segment, so 6 of each row's 16 codes are padding
    q_ref = np.empty((2, 96, 160), np.uint8)
    s_ref = np.empty((2, 6, 1, 16, 16), np.uint8)
    for i in range(2):
        q_ref[i], s_ref[i] = oracle.quant_weight_fp4(w[i])
    wd = torch.from_numpy(w).cuda()
    q = torch.empty((2, 96, 160), dtype=torch.uint8, device="cuda")
    s = torch.full((2, 6, 1, 16, 16), 0xAB, dtype=torch.uint8, device="cuda")  # padding must be cleared
    mdl.quantize_weight_fp4(wd, q, s)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_run_rejects_bad_arguments_without_launching():
    cfg = _cfg(4, 256, 8, 2, 128, 128)
    inp, w = data.build_layer(13, cfg)
    dinp, dw = gu.inputs_dev(inp), gu.weights_dev(w)
    h = _plan_for(cfg)
    try:
        out = torch.empty_like(dinp["x"])
        ptrs = [dinp["x"].data_ptr(), dinp["norm_w"].data_ptr(), dinp["gate_w"].data_ptr(),
                dinp["bias"].data_ptr()] + [dw[n].data_ptr() for n in gu.WEIGHT_NAMES] + [out.data_ptr()]
        assert mdl.run_ptrs(h, 0, ptrs) == mdl.EINVAL          # empty step
        assert mdl.run_ptrs(h, 5, ptrs) == mdl.EINVAL          # m > max_tokens
        for i in range(13):
            bad = list(ptrs)
            bad[i] = 0
            assert mdl.run_ptrs(h, 4, bad) == mdl.EINVAL       # null
            bad[i] = ptrs[i] + 8
            assert mdl.run_ptrs(h, 4, bad) == mdl.EINVAL       # misaligned
        alias = list(ptrs)
        alias[12] = ptrs[0]
        assert mdl.run_ptrs(h, 4, alias) == mdl.EINVAL         # out aliases x
        assert mdl.run_ptrs(h, 4, ptrs) == mdl.OK
        torch.cuda.synchronize()
    finally:
        mdl.destroy(h)


def test_plan_refuses_during_capture():
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    codes = []
    with torch.cuda.stream(s):
        g.capture_begin()
        try:
            torch.zeros(1, device="cuda").add_(1)  # keep the captured graph non-empty
            d = mdl.Dims(256, 8, 2, 128, 128, 4, 1e-6, 1.0)
            hh = mdl._P()
            codes.append(mdl.lib().moe_decode_plan(mdl.ctypes.byref(d), s.cuda_stream, mdl.ctypes.byref(hh)))
        finally:
            g.capture_end()
    assert codes == [mdl.ECAPTURE]


# ---------------------------------------------------------------- full size ----

_FULL = {}


def _full_layer(key, seed=0):
    """The full-size layers' seeded inputs for 48 rows and the weights of the
    experts the oracle picks for them (configs 1 and 2 use the first 1 and 16
    of those rows: their picks are among the 48 rows' picks).  One weight set
    is held at a time (8 GB of host memory at H = 5120, E = 256)."""
    want = (key, seed)
    if want not in _FULL:
        _FULL.clear()
        base = {"dsv41": synth.WORKLOADS[3], "draft": synth.WORKLOADS[4],
                "dsv41_fp4": dict(synth.WORKLOADS[3], routed="mxfp4")}[key]
        inp, w = data.build_layer(seed, base, experts="picked")
        _FULL[want] = (inp, w, gu.inputs_dev(inp), gu.weights_dev(w))
    return _FULL[want]


def _run_full(cfg, key, seed=0, rows_ref=None, schedule=None):
    """One step at full size planned exactly as bench.py plans it (max_tokens
    = m), every output row (or rows_ref) checked against the oracle."""
    inp_all, w, dinp_all, dw = _full_layer(key, seed)
    m = cfg["m"]
    inp = dict(inp_all, x=inp_all["x"][:m])
    dinp = dict(dinp_all, x=dinp_all["x"][:m].contiguous())
    h = _plan_for(cfg, max_tokens=m, schedule=schedule)
    try:
        out = gu.run(h, cfg, dinp, dw)
        torch.cuda.synchronize()
        print(f"[{cfg['name']} seed {seed}] ran; checking "
              f"{'every row' if rows_ref is None else rows_ref}", flush=True)
        _check_layer(cfg, h, inp, w, out, rows_ref=rows_ref)
    finally:
        mdl.destroy(h)


@pytest.mark.parametrize("idx", [5, 6])
def test_parity_tensor_parallel_share(idx):
    """One GPU's share of the layer under eight-way tensor parallelism (I = Is
    = 256 at the full hidden size and router): every output row."""
    cfg = synth.WORKLOADS[idx]
    inp, w = data.build_layer(0, cfg, experts="picked")
    dinp, dw = gu.inputs_dev(inp), gu.weights_dev(w)
    h = _plan_for(cfg, max_tokens=cfg["m"])
    try:
        out = gu.run(h, cfg, dinp, dw)
        torch.cuda.synchronize()
        print(f"[{cfg['name']}] ran; checking every row", flush=True)
        _check_layer(cfg, h, inp, w, out)
    finally:
        mdl.destroy(h)


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_parity_full_size(idx):
    _run_full(synth.WORKLOADS[idx], "dsv41")


@pytest.mark.parametrize("idx", [1])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_parity_full_size_persistent(idx, seed):
    """The persistent launch at full size, planned as bench.py plans it (and
    as its persistent figure plans it), against the oracle, on three seeds."""
    _run_full(dict(synth.WORKLOADS[idx], name=synth.WORKLOADS[idx]["name"] + "_persistent"), "dsv41",
              seed=seed, schedule="persistent")


def test_parity_full_size_m1_on_a_48_row_plan():
    """The M = 1 step on a plan made for 48 rows (a serving plan reused for
    every decode width): a sample row, as the plan changes only the layout."""
    cfg = synth.WORKLOADS[1]
    inp_all, w, dinp_all, dw = _full_layer("dsv41")
    inp = dict(inp_all, x=inp_all["x"][:1])
    dinp = dict(dinp_all, x=dinp_all["x"][:1].contiguous())
    h = _plan_for(cfg, max_tokens=48)
    try:
        out = gu.run(h, cfg, dinp, dw)
        torch.cuda.synchronize()
        _check_layer(cfg, h, inp, w, out)
    finally:
        mdl.destroy(h)


@pytest.mark.parametrize("idx", [1, 3])
@pytest.mark.parametrize("seed", [1, 2])
def test_parity_full_size_more_seeds(idx, seed):
    _run_full(synth.WORKLOADS[idx], "dsv41", seed=seed)


def test_parity_full_size_draft():
    _run_full(synth.WORKLOADS[4], "draft")


@pytest.mark.parametrize("idx", [1, 3])
def test_parity_full_size_mxfp4(idx):
    cfg = dict(synth.WORKLOADS[idx], routed="mxfp4", name=synth.WORKLOADS[idx]["name"] + "_fp4")
    _run_full(cfg, "dsv41_fp4")
    if idx == 3:
        _FULL.clear()
