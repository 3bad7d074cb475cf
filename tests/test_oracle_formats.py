"""Pins of the oracle's number formats against definitions outside the oracle.

E4M3 decode/encode, bf16 rounding, the E8M0 scale code and the MXFP8 row
quantiser (page "vllm.models.deepseek_v41.amd.mono.attention.device",
sections mx_code, mx_mul, fp8_pack4; page "vllm.models.deepseek_v41.amd.mono.
layer", section store_x8).  Every check here compares the oracle with
something other than itself: golden tables written from the format
definitions, brute-force nearest-value search, exact rational arithmetic or
torch's own conversions.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name, key_first):
    """Rows of a golden table: (first field, rest) or (all but last, last)."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                a, b = line.split(None, 1) if key_first else line.rsplit(None, 1)
                rows.append((a.strip(), b.strip()))
    return rows


# ---------------------------------------------------------------- E4M3 ----

def _e4m3_table():
    return np.array([oracle.e4m3_value(b) for b in range(256)])


def test_e4m3_golden_values():
    for byte, expr in _golden("e4m3_values.txt", True):
        want = eval(expr, {"math": math, "nan": float("nan")})
        got = oracle.e4m3_value(int(byte, 16))
        if math.isnan(want):
            assert math.isnan(got), byte
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), byte


def test_e4m3_decode_matches_torch():
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = t.to(torch.float64).numpy()
    got = _e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def _brute_force_e4m3(v):
    """Nearest of the 127 finite magnitudes by exhaustive distance, ties to the
    even code, sign bit from the input; |v| clamped to 448."""
    mags = np.array([oracle.e4m3_value(b) for b in range(0x7F)])
    a = np.minimum(np.abs(v), 448.0)
    d = np.abs(a[:, None] - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates prefer an even code
    even = cand & (np.arange(0x7F)[None, :] % 2 == 0)
    code = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (code | (np.signbit(v) * 0x80)).astype(np.uint8)


def test_e4m3_encode_brute_force_ties_and_neighbours():
    mags = np.array([oracle.e4m3_value(b) for b in range(0x7F)])
    mids = (mags[:-1] + mags[1:]) / 2  # exact ties
    f32 = mids.astype(np.float32)
    around = np.concatenate([
        mids, mags,
        np.nextafter(f32, np.float32(np.inf)).astype(np.float64),
        np.nextafter(f32, np.float32(0)).astype(np.float64),
        [0.0, 1e-30, 2.0 ** -10, 2.0 ** -10 * (1 + 2 ** -20), 447.9, 448.0, 460.0, 1e6],
    ])
    rng = np.random.default_rng(1)
    rand = rng.uniform(-450, 450, 200_000)
    tiny = rng.uniform(-2.0 ** -5, 2.0 ** -5, 50_000)
    v = np.concatenate([around, -around, rand, tiny, [-0.0]])
    assert np.array_equal(oracle.e4m3_rne_array(v), _brute_force_e4m3(v))


def test_e4m3_encode_matches_torch_on_fp32_grid():
    # every 61st fp32 bit pattern in [0, 448], both signs (about 37M values)
    bits = np.arange(0, 0x43E00001, 61, dtype=np.uint32)
    v = bits.view(np.float32).astype(np.float64)
    v = np.concatenate([v, -v])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_rne_array(v), ref)


# ---------------------------------------------------------------- bf16 ----

def test_bf16_rne_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(2)
    f = np.concatenate([
        rng.standard_normal(300_000).astype(np.float32),
        (rng.standard_normal(100_000) * 1e-38).astype(np.float32),  # subnormals
        rng.uniform(-3e38, 3e38, 10_000).astype(np.float32),
    ])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_rne_array(f.astype(np.float64)), ref)


def test_bf16_rne_single_rounding_from_double():
    # Closed forms: bf16 keeps 8 significant bits.
    cases = [
        (1.0 + 2.0 ** -8, 0x3F80),                 # tie -> even (1.0)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie -> even (1 + 2^-6)
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),    # above the tie: up; a detour
                                                   # through fp32 would tie to 1.0
        (-(1.0 + 2.0 ** -8 + 2.0 ** -40), 0xBF81),
        (2.0 ** -133, 0x0001),                     # smallest subnormal
        (2.0 ** -134, 0x0000),                     # tie with zero -> even
        (1.5 * 2.0 ** -134, 0x0001),
        (-0.0, 0x8000),
        (3.0e38 * 1.2, 0x7F80),                    # overflow
    ]
    for v, want in cases:
        assert oracle.bf16_rne_array(np.array([v]))[0] == want, v


# ---------------------------------------------------------------- E8M0 ----

def test_mx_code_hand_table():
    for expr, code in _golden("mx_code_table.txt", False):
        amax = eval(expr, {"math": math})
        assert oracle.mx_code(amax) == int(code), expr


def _code_exact(amax: float) -> int:
    """clamp(ceil(log2(max(amax, FLT_MIN) / 448)) + 127, 0, 254) in exact
    rational arithmetic."""
    q = Fraction(max(amax, 2.0 ** -126)) / 448
    j = q.numerator.bit_length() - q.denominator.bit_length()  # 2^(j-1) < q < 2^(j+1)
    while Fraction(2) ** j < q:
        j += 1
    while Fraction(2) ** (j - 1) >= q:
        j -= 1
    return min(max(j + 127, 0), 254)


def test_mx_code_matches_exact_formula():
    rng = np.random.default_rng(3)
    # random fp32 bit patterns over the whole positive finite range
    bits = rng.integers(0, 0x7F800000, 20_000, dtype=np.uint32)
    vals = list(bits.view(np.float32).astype(np.float64))
    for j in range(-148, 120):  # every boundary 448 * 2^j that is a finite fp32
        b = 448.0 * 2.0 ** j
        vals += [b, float(np.nextafter(np.float32(b), np.float32(np.inf))),
                 float(np.nextafter(np.float32(b), np.float32(0)))]
    vals = np.array(vals)
    got = oracle.mx_code_array(vals)
    want = np.array([_code_exact(float(v)) for v in vals])
    assert np.array_equal(got, want)


def test_mx_code_bracket_invariant():
    rng = np.random.default_rng(4)
    amax = np.abs(rng.standard_normal(50_000)) * 10.0 ** rng.uniform(-30, 30, 50_000)
    code = oracle.mx_code_array(amax)
    inner = (code > 0) & (code < 254)
    lo = 448.0 * np.exp2(code[inner] - 128.0)
    hi = 448.0 * np.exp2(code[inner] - 127.0)
    assert np.all(lo < amax[inner]) and np.all(amax[inner] <= hi)


def test_mx_multiplier_bit_identities():
    # [device] mx_mul / pow2 / rcp_pow2: the fp32 with bit pattern c << 23 is
    # 2^(c-127) for c in [1, 254]; (254 - c) << 23 is 2^(127-c) for c in [1, 253].
    for c in range(1, 255):
        f = np.array([c << 23], np.uint32).view(np.float32)[0]
        assert float(f) == 2.0 ** (c - 127)
    for c in range(1, 254):
        f = np.array([(254 - c) << 23], np.uint32).view(np.float32)[0]
        assert float(f) == 2.0 ** (127 - c)


# ------------------------------------------------------------ MXFP8 rows ----

def test_mx_quant_row_error_bound_and_top_element():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(32 * 400) * np.repeat(10.0 ** rng.uniform(-20, 20, 400), 32)
    q, codes = oracle.mx_quant_row(v)
    dq = np.array([oracle.e4m3_value(b) for b in q]) * np.exp2(np.repeat(codes.astype(float), 32) - 127)
    scaled = np.abs(v) * np.exp2(127.0 - np.repeat(codes.astype(float), 32))
    normal = scaled >= 2.0 ** -6          # E4M3 normal range: relative error <= 2^-4
    assert np.all(np.abs(dq - v)[normal] <= 2.0 ** -4 * np.abs(v)[normal])
    sub = ~normal                          # subnormal range: absolute error <= 2^-10
    assert np.all(np.abs(dq - v)[sub] * np.exp2(127.0 - np.repeat(codes.astype(float), 32))[sub] <= 2.0 ** -10)
    # the group's largest element lands in (224, 448] once scaled, and in
    # [224, 448] once rounded (224 is the E4M3 value just below 225)
    smax = scaled.reshape(-1, 32).max(axis=1)
    assert np.all((smax > 224.0) & (smax <= 448.0))
    top = np.abs(dq.reshape(-1, 32)).max(axis=1) * np.exp2(127.0 - codes)
    assert np.all((top >= 224.0) & (top <= 448.0))


def test_mx_quant_row_signed_zero_and_zero_group():
    v = np.zeros(64)
    v[3] = -1e-30   # rounds to zero in a group whose amax is 1.0
    v[4] = 1.0
    q, codes = oracle.mx_quant_row(v)
    assert codes[0] == 119 and codes[1] == 0
    # 1.0 * 2^(127 - 119) = 256 = 1.0 * 2^(15 - 7): byte 0.1111.000
    assert q[3] == 0x80 and q[0] == 0x00 and q[4] == 0x78
    assert np.all(q[32:] == 0)
