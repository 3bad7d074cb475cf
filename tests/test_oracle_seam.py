"""Pins of the oracle's seam functions around the MoE: the hyper-connection
residual fold and the attention seam's MXFP8 (page "vllm.models.deepseek_v41.
amd.mono.layer", sections run_ffn and store_x8; page "vllm.models.deepseek_v41.
amd.mono.runner", section DSV41MonoLayer.ffn for the shapes).  Each check
compares the oracle with something other than itself: a hand table of the
scale code, its equality with the MoE's code, exact cases where the
norm output is known in closed form (decoded through torch's float8_e4m3fn),
and mixes whose results are exact (identity, permutations, powers of two).
"""
import math
import os

import numpy as np
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "vllm_mx_code_table.txt")


def _bf16(v) -> np.ndarray:
    """Values exactly representable in bf16 -> their bit patterns."""
    a = np.asarray(v, np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _val(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------- scale code ----

def test_vllm_mx_code_hand_table():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                expr, code = line.rsplit(None, 1)
                rows.append((eval(expr, {"math": math}), int(code)))
    assert len(rows) >= 15
    for amax, code in rows:
        assert oracle.vllm_mx_code(amax) == code, (amax, code)


def test_vllm_code_equals_the_mx_code_and_brackets_amax():
    # the device page names mx_code as vLLM's ROCm MXFP8 scale code, so the
    # attention seam's code is the MoE's; either way the code is the smallest
    # c with amax <= 448 * 2^(c - 127): 448 * 2^(c - 128) < amax for c > 0
    rng = np.random.default_rng(4)
    amaxes = list(np.exp2(rng.uniform(-140, 128, 4000)))
    amaxes += [1.75 * 2.0 ** j * f for j in range(-130, 120, 7)
               for f in (1.0, 1.0 + 2.0 ** -30, 1.0 - 2.0 ** -30)]
    for amax in amaxes:
        amax = float(amax)
        v = oracle.vllm_mx_code(amax)
        assert v == oracle.mx_code(amax), amax
        if v < 254:
            assert amax <= math.ldexp(448.0, v - 127), amax
        if v > 0:
            assert amax > math.ldexp(448.0, v - 128), amax


# ------------------------------------------------- attention seam MXFP8 ----

def _e4m3_values(q) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(q, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_attn_x8_exact_norm_and_codes():
    # x = 1 everywhere and eps = 0: r = 1 exactly, so the norm output is the
    # weight row itself, chosen exactly representable
    H = 128
    w = np.ones(H, np.float32)
    w[0:32] = [500.0, -3.0, 1.0] + [0.25] * 29        # amax 500: code 128, scale 2^-1
    w[32:64] = [2.0, -1.5, 0.0] + [0.5] * 29          # amax 2: code 120, scale 2^7
    w[64:96] = 0.0                                    # zero group: code 0, zero bytes
    w[96:128] = [-448.0] + [7.0] * 31                 # amax 448: code 127, exact
    x8, x8s = oracle.attn_x8(_bf16(np.ones((1, H), np.float32)), _bf16(w), 0.0)
    assert list(x8s[0]) == [128, 120, 0, 127]
    got = _e4m3_values(x8[0])
    want = np.concatenate([
        [256.0, -1.5, 0.5] + [0.125] * 29,            # 250 rounds to 256 (240 | 256)
        np.array([2.0, -1.5, 0.0] + [0.5] * 29) * 128.0,
        np.zeros(32),
        [-448.0] + [7.0] * 31,
    ])
    assert np.array_equal(got, want)


def test_attn_x8_codes_values_and_error_bound():
    m, H = 3, 256
    x = synth.to_bf16_bits(synth.normal(3, 1, (m, H)))
    w = synth.to_bf16_bits(synth.normal(3, 2, (H,), 1.0, 0.1))
    x8, x8s = oracle.attn_x8(x, w, 1e-6)
    # the FFN seam's norm of the same rows is the attention norm rounded to
    # bf16; the attention codes follow mx_code's rule on the groups' amax
    y = _val(oracle.rmsnorm(x, w, 1e-6))
    for t in range(m):
        for g in range(H // 32):
            grp = y[t, 32 * g:32 * g + 32]
            c = int(x8s[t, g])
            amax_bf = np.abs(grp).max()
            # rounding to bf16 moves amax by at most 2^-8 relative
            assert oracle.vllm_mx_code(amax_bf * (1 - 2 ** -8)) <= c <= oracle.vllm_mx_code(amax_bf * (1 + 2 ** -8))
            dq = _e4m3_values(x8[t, 32 * g:32 * g + 32]) * 2.0 ** (c - 127)
            # within E4M3's half-ulp (2^-4 relative) of the value or half its
            # smallest step, plus the bf16 rounding of the comparison row;
            # the code keeps every scaled value within +-448, so the clamp
            # never bites
            err = np.abs(dq - grp)
            assert np.all(err <= np.abs(grp) * (2 ** -4 + 2 ** -8) + 2.0 ** (c - 127 - 10))


# ------------------------------------------------ hyper-connection fold ----

def _fold_inputs(seed, m, H):
    part = synth.to_bf16_bits(synth.normal(seed, 11, (m, H)))
    res_streams = synth.to_bf16_bits(synth.normal(seed, 12, (m, 4, H)))
    return part, res_streams


def test_hc_fold_identity_mix_keeps_the_streams():
    m, H = 2, 64
    part, r = _fold_inputs(1, m, H)
    post = np.zeros((m, 4), np.float32)
    res = np.tile(np.eye(4, dtype=np.float32), (m, 1, 1))
    pre = np.zeros((m, 4), np.float32)
    pre[:, 2] = 1.0
    ro, x = oracle.hc_fold(part, r, post, res, pre)
    assert np.array_equal(ro, r)
    assert np.array_equal(x, r[:, 2])                 # a one-hot pre picks a stream


def test_hc_fold_orientation_permutation_and_post():
    m, H = 2, 64
    part, r = _fold_inputs(2, m, H)
    perm = np.zeros((4, 4), np.float32)
    for i, j in enumerate([1, 2, 3, 0]):
        perm[i, j] = 1.0                              # output stream i takes input stream j
    res = np.tile(perm, (m, 1, 1))
    post = np.zeros((m, 4), np.float32)
    pre = np.zeros((m, 4), np.float32)
    pre[:, 0] = 1.0
    ro, x = oracle.hc_fold(part, r, post, res, pre)
    assert np.array_equal(ro[:, 0], r[:, 1]) and np.array_equal(ro[:, 3], r[:, 0])
    assert np.array_equal(x, r[:, 1])
    # no residual, powers of two on the attention output: exact scaled copies
    res0 = np.zeros((m, 4, 4), np.float32)
    post2 = np.tile(np.float32([1.0, 2.0, 0.5, -4.0]), (m, 1))
    ro2, x2 = oracle.hc_fold(part, r, post2, res0, pre)
    for i, f in enumerate([1.0, 2.0, 0.5, -4.0]):
        assert np.array_equal(_val(ro2[:, i]), _val(part) * f)
    assert np.array_equal(x2, part)


def test_hc_fold_linearity_in_powers_of_two():
    # doubling every mix doubles every output exactly
    m, H = 3, 96
    part, r = _fold_inputs(3, m, H)
    rng = np.random.default_rng(7)
    post = rng.uniform(0, 2, (m, 4)).astype(np.float32)
    res = rng.uniform(0, 1, (m, 4, 4)).astype(np.float32)
    pre = rng.uniform(0, 1, (m, 4)).astype(np.float32)
    ro, x = oracle.hc_fold(part, r, post, res, pre)
    ro2, _ = oracle.hc_fold(part, r, 2 * post, 2 * res, pre)
    assert np.array_equal(_val(ro2), 2 * _val(ro))
    _, x4 = oracle.hc_fold(part, r, post, res, 4 * pre)
    assert np.array_equal(_val(x4), 4 * _val(x))
