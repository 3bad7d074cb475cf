"""Parity of the seam upstream of the MoE with the oracle, through the C ABI:
the hyper-connection residual fold (new streams and input row) and the
attention seam's MXFP8, both bit-exact (the fold sums in double on both
sides and rounds once; the quantiser's decisions are integer)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

import moe_decode_layer_seam_amd as mdl  # noqa: E402


def _mixes(seed, m):
    rng = np.random.default_rng(seed)
    post = rng.uniform(0.0, 2.0, (m, 4)).astype(np.float32)
    res = rng.uniform(-0.5, 1.0, (m, 4, 4)).astype(np.float32)
    pre = rng.uniform(0.0, 1.0, (m, 4)).astype(np.float32)
    return post, res, pre


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("m,H", [(1, 256), (5, 640), (13, 5120), (48, 5120)])
def test_hc_fold_matches_oracle(m, H):
    part = synth.to_bf16_bits(synth.normal(40 + m, 11, (m, H)))
    resid = synth.to_bf16_bits(synth.normal(40 + m, 12, (m, 4, H)))
    post, res, pre = _mixes(m, m)
    ro_ref, x_ref = oracle.hc_fold(part, resid, post, res, pre)
    dpart, dres = gu.bf16_dev(part), gu.bf16_dev(resid.reshape(m * 4, H)).reshape(m, 4, H)
    ro, x = mdl.hc_fold(dpart, dres, torch.from_numpy(post).cuda(), torch.from_numpy(res).cuda(),
                        torch.from_numpy(pre).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(ro).reshape(m, 4, H), ro_ref)
    assert np.array_equal(_bits(x).reshape(m, H), x_ref)
    # in place: the new residual over the old one
    ro2, x2 = mdl.hc_fold(dpart, dres, torch.from_numpy(post).cuda(), torch.from_numpy(res).cuda(),
                          torch.from_numpy(pre).cuda(), residual_out=dres)
    torch.cuda.synchronize()
    assert ro2.data_ptr() == dres.data_ptr()
    assert np.array_equal(_bits(dres).reshape(m, 4, H), ro_ref)
    assert np.array_equal(_bits(x2).reshape(m, H), x_ref)


@pytest.mark.parametrize("m,H", [(1, 256), (7, 640), (48, 5120)])
def test_attn_x8_matches_oracle(m, H):
    x = synth.to_bf16_bits(synth.normal(50 + m, 1, (m, H)))
    if m > 1:
        x[1] = 0                                      # a zero row: every code 0
    spikes = synth.normal(50 + m, 5, (m, H // 32))
    xf = (np.asarray(x, np.uint32) << 16).view(np.float32).copy()
    xf[:, ::32] *= np.float32(1.0) + np.abs(spikes).astype(np.float32) * 8  # large first entries: varied codes
    x = (xf.view(np.uint32) >> 16).astype(np.uint16)
    w = synth.to_bf16_bits(synth.normal(50 + m, 2, (H,), 1.0, 0.1))
    x8_ref, x8s_ref = oracle.attn_x8(x, w, 1e-6)
    x8, x8s = mdl.attn_x8(gu.bf16_dev(x), gu.bf16_dev(w), 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(x8s.cpu().numpy(), x8s_ref)
    assert np.array_equal(x8.cpu().numpy(), x8_ref)
    # mx_code's bracket: the largest value of every nonzero group scales into
    # (224, 448], so its byte decodes to a magnitude in [224, 448]
    mag = torch.from_numpy(x8_ref & 0x7F).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    top = mag.reshape(m, H // 32, 32).max(axis=2)
    live = x8s_ref > 0
    assert live.any() and np.all((top[live] >= 224) & (top[live] <= 448))


def test_seam_entry_points_reject_bad_arguments():
    H = 256
    part = torch.zeros((2, H), dtype=torch.bfloat16, device="cuda")
    resid = torch.zeros((2, 4, H), dtype=torch.bfloat16, device="cuda")
    mix = torch.zeros((2, 4), dtype=torch.float32, device="cuda")
    res = torch.zeros((2, 4, 4), dtype=torch.float32, device="cuda")
    with pytest.raises(mdl.MoeDecodeError):
        mdl.hc_fold(part, resid, mix, res, mix, x=resid.view(-1)[:2 * H].view(2, H))  # x inside the residual
    with pytest.raises(mdl.MoeDecodeError):
        mdl.attn_x8(part, torch.zeros(H, dtype=torch.bfloat16, device="cuda"), -1.0)
