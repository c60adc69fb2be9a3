"""yarn_rope_table / yarn_rope_apply on the GPU vs the oracle."""
import numpy as np
import pytest
import torch

import long_context_attention_kv_amd as f4
import synth
from oracle import yarn as oyarn
from gpu_cases import bf16_tensor, bf16_values

pytestmark = pytest.mark.gpu

PROBES = [262144, 262145, 319999, 1048575]


def _params(factor, rd=256, mscale=0.0):
    return synth.YarnSpec(theta=1e7, rotary_dim=rd, factor=factor, orig_ctx=262144, beta_fast=32, beta_slow=1,
                          mscale=mscale)


def _gpu_params(s):
    return f4.YarnParams(s.theta, s.rotary_dim, s.factor, s.orig_ctx, s.beta_fast, s.beta_slow, s.mscale)


@pytest.mark.parametrize("factor", [1.0, 4.0, 1.220703125])
@pytest.mark.parametrize("rd", [256, 64])
def test_table_within_1e6(factor, rd):
    g = synth.rng(400, int(factor * 1000) + rd)
    pos = np.concatenate([[0, 1, 4095, 131071], PROBES, g.integers(0, 1 << 24, size=200)]).astype(np.int32)
    spec = _params(factor, rd)
    c, s = f4.yarn_rope_table(_gpu_params(spec), torch.from_numpy(pos).cuda())
    rc, rs = oyarn.yarn_table(spec, pos)
    torch.cuda.synchronize()
    assert np.max(np.abs(c.cpu().numpy() - rc)) <= 1e-6
    assert np.max(np.abs(s.cpu().numpy() - rs)) <= 1e-6


def test_table_explicit_mscale():
    spec = _params(4.0, mscale=1.5)
    pos = np.array(PROBES, np.int32)
    c, s = f4.yarn_rope_table(_gpu_params(spec), torch.from_numpy(pos).cuda())
    rc, rs = oyarn.yarn_table(spec, pos)
    assert np.max(np.abs(c.cpu().numpy() - rc)) <= 1e-6


def _ulp_bf16(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-38)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("rd", [256, 64])
def test_apply_bf16_within_one_ulp(rd):
    g = synth.rng(401, rd)
    T, H, D = 37, 16, 256
    bits = synth.f32_to_bf16_bits(synth.normal_f32(g, (T, H, D)))
    pos = g.integers(0, 1 << 20, size=T).astype(np.int32)
    spec = _params(4.0, rd)
    c, s = f4.yarn_rope_table(_gpu_params(spec), torch.from_numpy(pos).cuda())
    x = bf16_tensor(bits)
    y = f4.yarn_rope_apply(c, s, x)
    # oracle rotation in fp64 with the same fp32 table rows as inputs
    ref = oyarn.rope_apply(bf16_values(bits), c.cpu().numpy().astype(np.float64), s.cpu().numpy().astype(np.float64), rd)
    got = y.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= _ulp_bf16(ref) * 1.0001)
    # pass-through channels are copied exactly
    assert np.array_equal(got[..., rd:], bf16_values(bits)[..., rd:])


def test_apply_f32_in_place():
    g = synth.rng(402, 0)
    T, H, D, rd = 50, 4, 256, 256
    x = synth.normal_f32(g, (T, H, D))
    pos = g.integers(0, 1 << 20, size=T).astype(np.int32)
    spec = _params(4.0, rd)
    c, s = f4.yarn_rope_table(_gpu_params(spec), torch.from_numpy(pos).cuda())
    xt = torch.from_numpy(x.copy()).cuda()
    f4.yarn_rope_apply(c, s, xt, y=xt)
    ref = oyarn.rope_apply(x.astype(np.float64), c.cpu().numpy().astype(np.float64), s.cpu().numpy().astype(np.float64), rd)
    got = xt.cpu().numpy().astype(np.float64)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= ulp)


def test_table_plus_apply_vs_oracle_end_to_end():
    # GPU table + GPU rotation vs the oracle's fp64 table and rotation
    g = synth.rng(403, 0)
    T, H, D = 16, 16, 256
    bits = synth.f32_to_bf16_bits(synth.normal_f32(g, (T, H, D)))
    pos = np.array(PROBES * 4, np.int32)
    spec = _params(4.0)
    c, s = f4.yarn_rope_table(_gpu_params(spec), torch.from_numpy(pos).cuda())
    y = f4.yarn_rope_apply(c, s, bf16_tensor(bits)).float().cpu().numpy()
    rc, rs = oyarn.yarn_table(spec, pos)
    ref = oyarn.rope_apply(bf16_values(bits), rc, rs, 256)
    assert np.all(np.abs(y - ref) <= 2 * _ulp_bf16(ref))
