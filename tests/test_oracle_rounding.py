"""Pins of the oracle's rounding chains, bit for bit.

The RMSNorm feeding the MoE (page "vllm.models.deepseek_v41.amd.mono.layer",
sections run_ffn and store_normed: the seam's norm row stored as bf16) and
the hyper-connection fold (same page, run_ffn; shapes from page "vllm.models.
deepseek_v41.amd.mono.runner", DSV41MonoLayer.ffn) are compared here with
the chains of roundings their readings state, evaluated in exact rational
arithmetic (``tests/exact.py``):

  norm:  r = f32(1 / sqrt(ss / H + eps)) (the sqrt and divide in double);
         y = bf16(f32(f32(x r) w))
  fold:  stream i = bf16(sum_j res[i][j] r_j + post[i] part), the sum in
         double in that order; x = bf16(sum_i pre[i] stream_i) likewise.

A whole-tensor check compares every element with a vectorised evaluation of
the same chain in which every product is exact in double (so numpy's float32
cast is the chain's fp32 rounding).  Then, on the elements that lie next to a
bf16 rounding boundary, each plausible slip -- r kept in double, the
products in the other order, a dropped fp32 rounding, rounding through fp32
before bf16, an fp32 accumulator -- is evaluated exactly as well, and the
test requires that it changes at least one element's bits there while the
oracle keeps the stated chain's bits.  So any one of those slips in the
oracle fails this file.
"""
import math
from fractions import Fraction

import numpy as np

import oracle
import synth
from tests import exact
from tests.exact import BF16, F32, F64, rn


def _bf16_of_f32(y32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (finite values)."""
    u = y32.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_of_f64(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, one round to nearest even (values that are 0 or
    normal in bf16)."""
    v = np.asarray(v, np.float64)
    u = v.view(np.uint64)
    sign = (u >> 63).astype(np.uint64)
    mag = u & np.uint64(0x7FFFFFFFFFFFFFFF)
    # keep 7 of the 52 fraction bits: round at bit 45, ties to even
    r = (mag + np.uint64((1 << 44) - 1) + ((mag >> np.uint64(45)) & np.uint64(1))) >> np.uint64(45)
    exp = (r >> np.uint64(7)).astype(np.int64) - 1023 + 127
    frac = (r & np.uint64(0x7F)).astype(np.int64)
    bits = np.where(mag == 0, 0, (exp << 7) | frac).astype(np.int64)
    assert np.all((mag == 0) | ((exp >= 1) & (exp <= 254)))
    return (bits | (sign.astype(np.int64) << 15)).astype(np.uint16)


def _vals(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _near_bf16_boundary(y32: np.ndarray, ulps: int) -> np.ndarray:
    """Elements whose fp32 value lies within `ulps` fp32 steps of a bf16
    rounding midpoint."""
    low = y32.astype(np.float32).view(np.uint32) & 0xFFFF
    return np.abs(low.astype(np.int64) - 0x8000) <= ulps


# ------------------------------------------------------------- RMSNorm ----

def _norm_rows(m, H, seed):
    # N(0,1) rows with every |x| >= 2^-4, so each x^2 is a multiple of 2^-22
    # below 2^6: the sum of squares is exact in double in any order
    xf = synth.normal(seed, 1, (m, H))
    xf = np.where(np.abs(xf) < 2.0 ** -4, np.copysign(np.float32(2.0 ** -4), xf), xf)
    x = synth.to_bf16_bits(xf)
    w = synth.to_bf16_bits(synth.normal(seed, 2, (H,), 1.0, 0.1))
    return x, w


def _norm_scale(xrow_vals: np.ndarray, H: int, eps32: float) -> tuple[float, Fraction]:
    """(r in double, r rounded to fp32) for one row, the sum of squares exact."""
    ss = sum(Fraction(float(v)) ** 2 for v in xrow_vals)
    ss_f = float(ss)
    assert Fraction(ss_f) == ss
    r64 = 1.0 / math.sqrt(ss_f / H + eps32)        # IEEE double: / + sqrt / (each rounded once)
    return r64, rn(Fraction(r64), F32)


def test_rmsnorm_chain_bit_for_bit_and_slips_are_caught():
    m, H = 384, 4096
    eps32 = float(np.float32(1e-6))
    x, w = _norm_rows(m, H, 21)
    got = oracle.rmsnorm(x, w, 1e-6)
    xv, wv = _vals(x), _vals(w)

    r64s, r32s = [], []
    for t in range(m):
        r64, r32 = _norm_scale(xv[t], H, eps32)
        r64s.append(r64)
        r32s.append(r32)
    r32v = np.array([float(r) for r in r32s])[:, None]
    # x r: 8 x 24 significant bits, exact in double; f32 cast = the chain's rounding
    xa = (xv * r32v).astype(np.float32)
    # f32(x r) w: 24 x 8 bits, exact in double
    y32 = (xa.astype(np.float64) * wv[None, :]).astype(np.float32)
    want = _bf16_of_f32(y32)
    assert np.array_equal(got, want)

    # the elements where a slip of one or two fp32 steps can show
    cand = np.argwhere(_near_bf16_boundary(y32, 6))
    assert len(cand) > 100
    slips = {
        "r kept in double": lambda X, W, t: rn(rn(rn(X * Fraction(r64s[t]), F32) * W, F32), BF16),
        "(x w) r instead of (x r) w": lambda X, W, t: rn(rn(rn(X * W, F32) * r32s[t], F32), BF16),
        "one fp32 rounding of x r w": lambda X, W, t: rn(rn(X * r32s[t] * W, F32), BF16),
        "f32(x r) w rounded straight to bf16": lambda X, W, t: rn(rn(X * r32s[t], F32) * W, BF16),
        "whole chain in double": lambda X, W, t: rn(rn(rn(X * Fraction(r64s[t]), F64) * W, F64), BF16),
    }
    caught = {k: 0 for k in slips}
    for t, i in cand:
        X, W = Fraction(float(xv[t, i])), Fraction(float(wv[i]))
        right = rn(rn(rn(X * r32s[t], F32) * W, F32), BF16)
        assert exact.bf16_bits(right) == int(got[t, i]) or right == 0
        for k, f in slips.items():
            if f(X, W, t) != right:
                caught[k] += 1
    assert all(n > 0 for n in caught.values()), caught


def test_rmsnorm_scale_rounded_once_from_double():
    # closed form: x = 3 everywhere, H = 4, eps = 0 gives r = RN64(1/3),
    # whose fp32 rounding 0x3EAAAAAB is 2^-25 / 3 above 1/3; then 3 r =
    # 1 + 2^-25 rounds to 1 in fp32, and with w = 1 + 2^-7 every y is
    # bf16(1 + 2^-7) exactly
    x = exact.bf16_bits(Fraction(3))
    w = exact.bf16_bits(Fraction(1) + Fraction(1, 128))
    got = oracle.rmsnorm(np.full((1, 4), x, np.uint16), np.full(4, w, np.uint16), 0.0)
    assert np.all(got == w)


# ------------------------------------------------- hyper-connection fold ----

def _fold_inputs(m, H, seed):
    part = synth.to_bf16_bits(synth.normal(seed, 11, (m, H)))
    resid = synth.to_bf16_bits(synth.normal(seed, 12, (m, 4, H)))
    rng = np.random.default_rng(seed)
    post = rng.uniform(0.0, 2.0, (m, 4)).astype(np.float32)
    res = rng.uniform(0.0, 1.0, (m, 4, 4)).astype(np.float32)
    pre = rng.uniform(0.0, 1.0, (m, 4)).astype(np.float32)
    return part, resid, post, res, pre


def test_hc_fold_chain_bit_for_bit_and_slips_are_caught():
    m, H = 64, 8192
    part, resid, post, res, pre = _fold_inputs(m, H, 31)
    ro, x = oracle.hc_fold(part, resid, post, res, pre)

    rv = _vals(resid)                          # [m, 4, H]
    pv = _vals(part)                           # [m, H]
    post64, res64, pre64 = post.astype(np.float64), res.astype(np.float64), pre.astype(np.float64)
    # numpy float64 elementwise operations in the stated order are the
    # double sums of the reading (each product of an fp32 and a bf16 is exact)
    acc = np.zeros((m, 4, H))
    for i in range(4):
        a = np.zeros((m, H))
        for j in range(4):
            a = a + res64[:, i, j, None] * rv[:, j]
        acc[:, i] = a + post64[:, i, None] * pv
    want_ro = _bf16_of_f64(acc)
    assert np.array_equal(ro, want_ro)
    xs = np.zeros((m, H))
    for i in range(4):
        xs = xs + pre64[:, i, None] * _vals(want_ro[:, i])
    assert np.array_equal(x, _bf16_of_f64(xs))

    # slips, each evaluated exactly on the elements next to a bf16 boundary
    near = _near_bf16_boundary(acc.astype(np.float32), 2)
    cand = np.argwhere(near)
    assert len(cand) > 20
    through_f32 = 0
    for t, i, c in cand:
        terms = [Fraction(float(res[t, i, j])) * Fraction(float(rv[t, j, c])) for j in range(4)]
        terms.append(Fraction(float(post[t, i])) * Fraction(float(pv[t, c])))
        s = Fraction(0)
        for term in terms:                     # the double sum of the reading
            s = rn(s + term, F64)
        right = rn(s, BF16)
        assert exact.bf16_bits(right) == int(ro[t, i, c]) or right == 0
        if rn(rn(s, F32), BF16) != right:
            through_f32 += 1
    assert through_f32 > 0

    # an fp32 accumulator, and x from the unrounded streams, differ often
    acc32 = np.zeros((m, 4, H), np.float32)
    for i in range(4):
        a = np.zeros((m, H), np.float32)
        for j in range(4):
            a = (a + (res[:, i, j, None] * rv[:, j].astype(np.float32))).astype(np.float32)
        acc32[:, i] = (a + post[:, i, None] * pv.astype(np.float32)).astype(np.float32)
    assert (_bf16_of_f32(acc32) != ro).sum() > 10
    xs_unrounded = np.zeros((m, H))
    for i in range(4):
        xs_unrounded = xs_unrounded + pre64[:, i, None] * acc[:, i]
    assert (_bf16_of_f64(xs_unrounded) != x).sum() > 100
