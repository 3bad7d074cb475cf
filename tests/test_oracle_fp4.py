"""Pins of the oracle's MXFP4 (A8W4) routed-expert path against things other
than itself: the E2M1 value table of the OCP MX specification (golden file),
brute-force nearest-value search over that table, hand-checked scale codes,
exactly representable weights, and the independent torch pipeline (which
decodes E2M1 through the golden table)."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import data
from tests import torch_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.txt")


def _golden():
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                nib, v = line.split()
                rows.append((int(nib, 16), float(v)))
    return rows


def test_e2m1_golden_values():
    rows = _golden()
    assert [n for n, _ in rows] == list(range(16))
    for nib, v in rows:
        got = oracle.e2m1_value(nib)
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), (nib, got, v)


def _nearest_even(v: float) -> int:
    """Brute force over the golden table: the nearest magnitude, ties to the
    code with a zero mantissa bit, |v| saturating at 6, sign kept."""
    mags = [(n, val) for n, val in _golden() if n < 8]
    a = min(abs(v), 6.0)
    best = min(mags, key=lambda nv: (abs(a - nv[1]), nv[0] & 1))
    return best[0] | (8 if math.copysign(1.0, v) < 0 else 0)


def test_e2m1_encode_brute_force_grid_and_ties():
    vals = [0.0, -0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 100.0, -0.25, -5.0, -1e-30]
    grid = np.linspace(-8.0, 8.0, 4097).tolist()
    for v in vals + grid:
        assert oracle.e2m1_rne(v) == _nearest_even(v), v
    # every value's neighbours either side of each midpoint
    for lo, hi in [(0.0, 0.5), (0.5, 1.0), (1.0, 1.5), (1.5, 2.0), (2.0, 3.0), (3.0, 4.0), (4.0, 6.0)]:
        mid = (lo + hi) / 2
        for v in (np.nextafter(mid, -np.inf), mid, np.nextafter(mid, np.inf)):
            assert oracle.e2m1_rne(float(v)) == _nearest_even(float(v)), v
    arr = np.array(grid)
    assert np.array_equal(oracle.e2m1_rne_array(arr), np.array([_nearest_even(v) for v in grid], np.uint8))


def test_fp4_code_hand_table_and_bracket():
    # the smallest c with amax <= 6 * 2^(c - 127), checked by hand
    table = [(0.0, 0), (1e-40, 0), (6 * 2.0 ** -127, 0), (6 * 2.0 ** -126, 1), (6.0, 127),
             (float(np.nextafter(6.0, 7.0)), 128), (3.0, 126), (3.0000001, 127), (12.0, 128),
             (1.0, 125), (0.75, 124), (1e38, 251), (3e38, 253)]
    for amax, code in table:
        assert oracle.fp4_code(amax) == code, (amax, code)
    rng = np.random.default_rng(3)
    for amax in np.exp(rng.uniform(-80, 80, 2000)):
        c = oracle.fp4_code(float(amax))
        if 0 < c < 254:
            assert 6.0 * 2.0 ** (c - 128) < amax <= 6.0 * 2.0 ** (c - 127)


def test_fp4_quantiser_layout_and_nearest_values():
    rng = np.random.default_rng(5)
    w = rng.normal(0.0, 0.02, (64, 96)).astype(np.float32)
    w[3, 32:64] = 0.0                                    # an all-zero block: code 0
    w[7, :32] = np.float32([0.5, 1, 1.5, 2, 3, 4, 6, -6] * 4)  # exact at code 127
    q, sb = oracle.quant_weight_fp4(w)
    # blocked codes: [row tile of 16][512-column segment][row in tile][32-column block in segment]
    assert q.shape == (64, 48) and sb.shape == (4, 1, 16, 16)
    assert np.all(sb[:, :, :, 3:] == 0)                  # padding past the 3 real blocks
    s = sb.transpose(0, 2, 1, 3).reshape(64, 16)[:, :3]  # back to [row, block]
    assert s[3, 1] == 0 and np.all(q[3, 16:32] == 0)
    assert s[7, 0] == 127
    assert list(q[7, :4]) == [0x21, 0x43, 0x65, 0xF7]    # column 2i in the low nibble
    table = dict(_golden())
    for r in range(64):
        for b in range(3):
            blk = w[r, 32 * b:32 * b + 32].astype(np.float64)
            code = int(s[r, b])
            assert code == sb[r // 16, 0, r % 16, b]
            assert code == oracle.fp4_code(float(np.abs(blk).max()))
            scale = 2.0 ** (127 - code)
            for i in range(32):
                byte = q[r, 16 * b + i // 2]
                nib = (byte >> 4) if i & 1 else (byte & 0xF)
                assert nib == _nearest_even(blk[i] * scale), (r, b, i)
                # dequantised value within half a spacing (at most 1 unit at 2^(code-127))
                assert abs(table[nib] / scale - blk[i]) <= 1.0 / scale


def test_fp4_blocked_code_order():
    # cols 1056: two whole 512-column segments and one of 32 columns, so each
    # row tile holds three 256-byte blocks, the last with 15 padding columns
    rows, cols = 48, 1056
    w = np.zeros((rows, cols), np.float32)
    for r in range(rows):
        for b in range(cols // 32):
            w[r, 32 * b + (r + b) % 32] = 6.0 * 2.0 ** ((r * 7 + b * 3) % 40 - 20)
    q, sb = oracle.quant_weight_fp4(w)
    assert sb.shape == (3, 3, 16, 16)
    flat = sb.reshape(-1)
    seen = set()
    for r in range(rows):
        for b in range(cols // 32):
            pos = ((r // 16) * 3 + b // 16) * 256 + (r % 16) * 16 + b % 16
            assert oracle.fp4_code_index(cols, r, b) == pos
            assert flat[pos] == 127 + (r * 7 + b * 3) % 40 - 20, (r, b)
            seen.add(pos)
    pad = np.ones(flat.size, bool)
    pad[list(seen)] = False
    assert pad.sum() == 3 * 15 * 16 and np.all(flat[pad] == 0)


def test_fp4_unit_scale_round_trip_and_plain_matmul():
    # codes 127 and exactly representable values: quantising loses nothing, so
    # the expert's products are those of the plain fp64 matmul of the inputs
    H, I = 64, 32
    rng = np.random.default_rng(9)
    xvals = rng.choice([0.5, 1.0, -1.0, 2.0, 0.25], H)
    xvals[0] = xvals[32] = 2.0
    x8, x8s = oracle.mx_quant_row(xvals)
    assert np.all(x8s == oracle.mx_code(2.0))
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    w13f = rng.choice(mags, (2 * I, H)) * rng.choice([-1.0, 1.0], (2 * I, H))
    w13f[:, 0] = w13f[:, 32] = 6.0  # every block's amax is 6: code 127
    w2f = rng.choice(mags, (H, I))
    w2f[:, 0] = 6.0
    q13, s13 = oracle.quant_weight_fp4(w13f.astype(np.float32))
    q2, s2 = oracle.quant_weight_fp4(w2f.astype(np.float32))
    assert np.all(s13[..., :2] == 127) and np.all(s2[..., :1] == 127)  # the real blocks
    assert np.all(s13[..., 2:] == 0) and np.all(s2[..., 1:] == 0)      # padding
    assert np.array_equal(torch_ref.fp4_dequant(q13, s13).numpy(), w13f)
    assert np.array_equal(torch_ref.fp4_dequant(q2, s2).numpy(), w2f)
    got = oracle.expert(x8, x8s, q13, s13, q2, s2, fmt="mxfp4")
    xd = torch_ref.mx_dequant(torch.from_numpy(x8), torch.from_numpy(x8s))
    h = torch.from_numpy(w13f) @ xd
    a = (torch.nn.functional.silu(h[:I]) * h[I:]).to(torch.float32).to(torch.float64)
    aq, ac = torch_ref.mx_quant(a)
    y = torch.from_numpy(w2f) @ torch_ref.mx_dequant(aq, ac)
    assert np.array_equal(got["a8s"], ac.numpy())
    assert np.allclose(got["y"], y.numpy(), rtol=1e-12, atol=0)


def test_fp4_expert_matches_torch_reference():
    H, I = 256, 128
    x = synth.normal(21, 1, (H,))
    x8, x8s = oracle.mx_quant_row(x)
    q13, s13 = oracle.quant_weight_fp4(synth.expert_f32(21, "w13", 0, 2 * I, H))
    q2, s2 = oracle.quant_weight_fp4(synth.expert_f32(21, "w2", 0, H, I))
    got = oracle.expert(x8, x8s, q13, s13, q2, s2, fmt="mxfp4")
    y, aq, ac = torch_ref.expert(torch.from_numpy(x8), torch.from_numpy(x8s), q13, s13, q2, s2, "mxfp4")
    assert np.array_equal(got["a8s"], ac.numpy())
    assert (got["a8"] == aq.numpy()).mean() > 0.99
    assert np.allclose(got["y"], y.numpy(), rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("m", [1, 3])
def test_fp4_layer_matches_torch_reference(m):
    cfg = dict(synth.WORKLOADS[0], routed="mxfp4", m=m)
    inp, w = data.build_layer(4, cfg)
    dims = data.dims_of(cfg)
    o = oracle.layer(dims, inp, w)
    r = torch_ref.layer(dims, inp, w, o["normed"])
    assert np.array_equal(o["ids"], r["ids"])
    assert np.allclose(o["out_f64"], r["out_f64"], rtol=1e-9, atol=1e-12)


def test_fp4_scale_plus_one_doubles_the_expert_exactly():
    H, I = 128, 64
    x8, x8s = oracle.mx_quant_row(synth.normal(22, 1, (H,)))
    q13, s13 = oracle.quant_weight_fp4(synth.expert_f32(22, "w13", 0, 2 * I, H))
    q2, s2 = oracle.quant_weight_fp4(synth.expert_f32(22, "w2", 0, H, I))
    a = oracle.expert(x8, x8s, q13, s13, q2, s2, fmt="mxfp4")
    b = oracle.expert(x8, x8s, q13, s13, q2, (s2 + 1).astype(np.uint8), fmt="mxfp4")
    assert np.array_equal(b["y"], 2 * a["y"])
