"""kv_cache_write_f4 on the GPU vs the oracle: nibbles and fp16 scales bit for bit."""
import numpy as np
import pytest
import torch

import long_context_attention_kv_amd as f4
import synth
from oracle import f4 as of4
from gpu_cases import PagedSet, cache_arrays_equal

pytestmark = pytest.mark.gpu


def _write_both(k, v, slots, P, H, D):
    oc = of4.Cache(P, H, D)
    oc.write(k, v, slots)
    gc = f4.F4Cache(P, H, D)
    f4.kv_cache_write_f4(gc, torch.from_numpy(np.ascontiguousarray(k)).cuda(),
                         torch.from_numpy(np.ascontiguousarray(v)).cuda(),
                         torch.from_numpy(np.asarray(slots, np.int32)).cuda())
    torch.cuda.synchronize()
    return gc, oc


@pytest.mark.parametrize("T,H,D,P", [(1, 1, 32, 1), (5, 2, 64, 2), (130, 4, 256, 4), (64 * 9 + 7, 4, 256, 12)])
def test_random_slots_bit_exact(T, H, D, P):
    g = synth.rng(300, T)
    k = synth.normal_f32(g, (T, H, D))
    v = synth.normal_f32(g, (T, H, D)) * np.float32(3.0)
    slots = g.permutation(P * 64)[:T].astype(np.int32)
    slots[::7] = -1
    gc, oc = _write_both(k, v, slots, P, H, D)
    assert cache_arrays_equal(gc, oc) == []


def test_edge_values_bit_exact():
    # zero blocks, subnormal scales, saturating scales, exact ties and near ties
    g = synth.rng(301, 0)
    T, H, D, P = 64, 2, 256, 1
    k = synth.normal_f32(g, (T, H, D))
    v = synth.normal_f32(g, (T, H, D))
    k[0, 0, :32] = 0.0
    k[1, 0, :32] *= np.float32(1e-6)
    k[2, 0, :32] *= np.float32(1e-9)
    k[3, 0, :32] = np.float32(7e5)
    k[3, 0, 5] = np.float32(-1e6)
    # ties: s = 1 exactly (absmax 8), values at k + 1/2 and one ulp either side
    row = np.array([8.0] + [(j % 16 - 8) + 0.5 for j in range(31)], dtype=np.float32)
    k[4, 1, :32] = row
    k[5, 1, :32] = np.nextafter(row, np.float32(np.inf))
    k[6, 1, :32] = np.nextafter(row, np.float32(-np.inf))
    v[7, 1, 32:64] = -row
    for t in range(8, 40):
        s = np.float16(g.uniform(1e-3, 50.0))
        base = (np.arange(32) % 16 - 8 + 0.5) * np.float64(s)
        x = base.astype(np.float32)
        x = np.nextafter(x, np.float32(np.inf) if t % 2 else np.float32(-np.inf))
        x[0] = np.float32(8 * np.float64(s))
        k[t, 0, 64:96] = x
    slots = np.arange(T, dtype=np.int32)
    gc, oc = _write_both(k, v, slots, P, H, D)
    assert cache_arrays_equal(gc, oc) == []


def test_skip_and_overwrite():
    g = synth.rng(302, 0)
    T, H, D, P = 70, 4, 256, 2
    k = synth.normal_f32(g, (T, H, D))
    v = synth.normal_f32(g, (T, H, D))
    slots = np.full(T, -1, np.int32)
    slots[10:20] = np.arange(100, 110)
    gc, oc = _write_both(k, v, slots, P, H, D)
    assert cache_arrays_equal(gc, oc) == []
    # overwrite part of it with new values
    k2 = synth.normal_f32(g, (T, H, D))
    v2 = synth.normal_f32(g, (T, H, D))
    s2 = np.full(T, -1, np.int32)
    s2[:5] = [105, 0, 63, 64, 127]
    oc.write(k2, v2, s2)
    f4.kv_cache_write_f4(gc, torch.from_numpy(k2).cuda(), torch.from_numpy(v2).cuda(), torch.from_numpy(s2).cuda())
    torch.cuda.synchronize()
    assert cache_arrays_equal(gc, oc) == []


def test_config0_shape_bit_exact():
    ps = PagedSet([4096], Hkv=4, D=256, seed=1)
    assert cache_arrays_equal(ps.gc, ps.oc) == []


def test_outlier_channels_bit_exact():
    ps = PagedSet([1000, 333], Hkv=4, D=256, seed=2, outliers=True)
    assert cache_arrays_equal(ps.gc, ps.oc) == []


def test_determinism():
    g = synth.rng(303, 0)
    T, H, D, P = 200, 4, 256, 4
    k = synth.normal_f32(g, (T, H, D))
    v = synth.normal_f32(g, (T, H, D))
    slots = g.permutation(P * 64)[:T].astype(np.int32)
    a, _ = _write_both(k, v, slots, P, H, D)
    b, _ = _write_both(k, v, slots, P, H, D)
    for x, y in ((a.k_nib, b.k_nib), (a.v_nib, b.v_nib), (a.k_scale, b.k_scale), (a.v_scale, b.v_scale)):
        assert torch.equal(x, y)
