"""End-to-end check of the key path: the GPU's YaRN table (stored in fp32),
rotation and F4 write against the oracle's own fp64 table, fp64 rotation,
rounding to fp32 and quantisation.  The two pipelines round the rotated keys
differently (the table's fp32 rows vs exact fp64), so a key that lands within
an fp32 rounding of a code boundary can take the neighbouring code: the test
counts those nibble flips and checks that each is a single step at a boundary
and that they are rare.  It is a characterisation of the pipeline, reported,
beside the bit-exact writer test (same fp32 inputs on both sides)."""
import numpy as np
import pytest
import torch

import long_context_attention_kv_amd as f4
import synth
from oracle import f4 as of4
from oracle import yarn as oyarn

pytestmark = pytest.mark.gpu

PAGE, HKV, D = 64, 4, 256


def test_nibble_flips_of_the_fp32_table_pipeline():
    n, t0 = 65536, 262144  # positions past the original context
    print(f"end to end: {n} keys at positions {t0}..{t0 + n - 1}, YaRN x4", flush=True)
    g = synth.rng(960, 0)
    k = synth.normal_f32(g, (n, HKV, D))
    v = synth.normal_f32(g, (n, HKV, D))
    spec = synth.YarnSpec(factor=4.0)
    pos = np.arange(t0, t0 + n)
    slots = np.arange(n, dtype=np.int32)  # page p holds tokens 64p .. 64p + 63
    # GPU: fp32 table rows, rotation, F4 write
    yp = f4.YarnParams(spec.theta, spec.rotary_dim, spec.factor, spec.orig_ctx, spec.beta_fast, spec.beta_slow,
                       spec.mscale)
    c, s = f4.yarn_rope_table(yp, torch.from_numpy(pos.astype(np.int32)).cuda())
    kt = f4.yarn_rope_apply(c, s, torch.from_numpy(k).cuda())
    gc = f4.F4Cache(n // PAGE, HKV, D)
    f4.kv_cache_write_f4(gc, kt, torch.from_numpy(v).cuda(), torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    # oracle: its own fp64 table and rotation, one rounding to fp32, its quantiser
    cs, sn = oyarn.yarn_table(spec, pos)
    kr = oyarn.rope_apply(k.astype(np.float64), cs, sn, spec.rotary_dim).astype(np.float32)
    oc = of4.Cache(n // PAGE, HKV, D)
    oc.write(kr, v, slots)

    gk = gc.k_nib.cpu().numpy()
    ok, oks, ov, ovs = oc.arrays()
    assert np.array_equal(gc.v_nib.cpu().numpy(), ov), "values take no rotation: bit-exact"
    assert np.array_equal(gc.v_scale.cpu().numpy().view(np.uint16), ovs)
    g_codes = of4.unpack_block_bytes(gk).astype(np.int16)
    o_codes = of4.unpack_block_bytes(ok).astype(np.int16)
    flips = int(np.count_nonzero(g_codes != o_codes))
    scale_diff = int(np.count_nonzero(gc.k_scale.cpu().numpy().view(np.uint16) != oks))
    total = g_codes.size
    step = np.abs(g_codes - o_codes)
    print(f"end to end: {flips} of {total} key nibbles differ ({flips / total:.2e}); "
          f"{scale_diff} of {oks.size} key scales differ", flush=True)
    # where the block scale agrees, a flip is one code step, from a rounding boundary
    eq = gc.k_scale.cpu().numpy().view(np.uint16) == oks               # [P][H][64][D/32]
    same_scale = np.broadcast_to(eq.transpose(0, 1, 3, 2)[..., None], g_codes.shape)  # codes [P][H][D/32][64][32]
    assert step[same_scale].max(initial=0) <= 1
    assert flips <= 1e-3 * total and scale_diff <= 1e-3 * oks.size
