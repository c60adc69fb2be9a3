"""paged_attn_decode_step_f4 (the new token of each sequence rotated and written,
then the decode, in one call) on the GPU: bit for bit the results of the
separate entry points (yarn_rope_apply on q and on k, kv_cache_write_f4,
paged_attn_decode_f4), and against the oracle (its rotation with the same fp32
table rows, its quantiser and its attention) within 2e-3 x output RMS."""
import numpy as np
import pytest
import torch

import long_context_attention_kv_amd as f4
import synth
from oracle import attention as oatt
from oracle import f4 as of4
from oracle import yarn as oyarn
from gpu_cases import PagedSet, assert_attention_close, assert_states_close, bf16_tensor, bf16_values

pytestmark = pytest.mark.gpu
SM = 1.0 / 16.0
PAGE, D = 64, 256


def clone_cache(gc: f4.F4Cache) -> f4.F4Cache:
    c2 = f4.F4Cache(gc.num_pages, gc.num_kv_heads, gc.head_dim, v_scale_per_token=gc.v_scale_per_token)
    for name in ("k_nib", "k_scale", "v_nib", "v_scale"):
        getattr(c2, name).copy_(getattr(gc, name))
    return c2


def run_step(lengths, seed, Hkv=4, G=4, rotary_dim=256, v_per_token=False, skip=(), factor=4.0, W=1, wt=0):
    """The cache holds every token of each sequence; the step rewrites the last
    one (position n - 1) from new fp32 K / V and decodes over all n."""
    print(f"decode step: lengths={lengths} Hkv={Hkv} G={G} rotary_dim={rotary_dim} v_per_token={v_per_token} "
          f"skip={skip} W={W}", flush=True)
    ps = PagedSet(lengths, Hkv=Hkv, seed=seed, outliers=True, v_per_token=v_per_token)
    B, Hq = len(lengths), G * Hkv
    g = synth.rng(700 + seed, 2)
    qbits = synth.f32_to_bf16_bits(synth.normal_f32(g, (B, Hq, D)))
    k_new = synth.normal_f32(g, (B, Hkv, D))
    v_new = synth.normal_f32(g, (B, Hkv, D))
    pos = np.array([n - 1 for n in lengths], dtype=np.int64)
    slots = np.array([ps.pt[b, p // PAGE] * PAGE + p % PAGE for b, p in enumerate(pos)], dtype=np.int32)
    for b in skip:
        slots[b] = -1
    spec = synth.YarnSpec(factor=factor, rotary_dim=rotary_dim)
    yp = f4.YarnParams(spec.theta, spec.rotary_dim, spec.factor, spec.orig_ctx, spec.beta_fast, spec.beta_slow,
                       spec.mscale)
    cos, sin = f4.yarn_rope_table(yp, torch.from_numpy(pos.astype(np.int32)).cuda())
    q, kn, vn = bf16_tensor(qbits), torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda()
    sl, pt, lens = torch.from_numpy(slots).cuda(), ps.gpu_page_table(), ps.gpu_lengths()
    inputs = [t.clone() for t in (q, kn, vn)]
    max_ctx = max(lengths)

    # the separate entry points, on a copy of the cache
    gc2 = clone_cache(ps.gc)
    q_rot = f4.yarn_rope_apply(cos, sin, q)
    k_rot = f4.yarn_rope_apply(cos, sin, kn)
    f4.kv_cache_write_f4(gc2, k_rot, vn, sl)
    ref = f4.paged_attn_decode_f4(gc2, q_rot, pt, lens, max_ctx, SM, num_windows=W, window_tokens=wt)
    got = f4.paged_attn_decode_step_f4(ps.gc, cos, sin, q, kn, vn, sl, pt, lens, max_ctx, SM, num_windows=W,
                                       window_tokens=wt)
    torch.cuda.synchronize()
    for a, b, what in zip(got, ref, ("out", "m", "l")):
        assert torch.equal(a, b), f"step vs separate calls: {what}"
    for name in ("k_nib", "k_scale", "v_nib", "v_scale"):
        assert torch.equal(getattr(ps.gc, name), getattr(gc2, name)), f"step vs separate calls: cache {name}"
    for a, b in zip((q, kn, vn), inputs):
        assert torch.equal(a, b), "the step leaves its inputs unchanged"

    # oracle: the same fp32 table rows, its own rotation, quantiser and attention
    cs, sn = cos.cpu().numpy().astype(np.float64), sin.cpu().numpy().astype(np.float64)
    qr = of4.bf16_round(oyarn.rope_apply(bf16_values(qbits), cs, sn, rotary_dim))
    kr = oyarn.rope_apply(k_new.astype(np.float64), cs, sn, rotary_dim).astype(np.float32)
    ps.oc.write(kr, v_new, slots)
    ro, rm, rl = oatt.decode(ps.oc, qr, ps.pt, ps.lengths, SM, window_tokens=wt, num_windows=W)
    o, m, l = (x.cpu().numpy() for x in got)
    assert_attention_close(o, ro, "decode step vs oracle")
    assert_states_close(m, l, rm, rl, "decode step vs oracle")
    return ps, slots


def test_step_matches_separate_calls_and_oracle():
    run_step([700, 130, 64 * 20 + 5], seed=1)


def test_step_new_token_opens_a_page_and_partial_rotation():
    # the new token is the first of its page (n - 1 = 64 k); only half the channels rotate
    run_step([65, 129, 1000], seed=2, rotary_dim=128)


def test_step_skipped_slot_and_v_per_token():
    # slot -1: that sequence's token is not written (its cache keeps the old cells)
    ps, slots = run_step([300, 77], seed=3, v_per_token=True, skip=(1,))
    assert slots[1] == -1


@pytest.mark.parametrize("G,Hkv", [(1, 4), (2, 2), (8, 2)])
def test_step_other_groups(G, Hkv):
    run_step([500, 1], seed=10 + G, Hkv=Hkv, G=G)


def test_step_with_windows_and_plain_rope():
    run_step([3000, 640], seed=4, factor=1.0, W=3, wt=1024)
