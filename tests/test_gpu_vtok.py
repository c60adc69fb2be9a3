"""The per-token V scale variant (one fp16 V scale per token and head) on the GPU
vs the oracle: the writer bit for bit, decode and prefill to max |delta| <= 2e-3
x output RMS."""
import numpy as np
import pytest
import torch

import long_context_attention_kv_amd as f4
import synth
from oracle import f4 as of4
from gpu_cases import (PagedSet, assert_attention_close, assert_states_close, bf16_tensor, cache_arrays_equal,
                       oracle_decode, random_q)
from test_gpu_prefill import Chunk

pytestmark = pytest.mark.gpu
SM = 1.0 / 16.0


def _write_both(k, v, slots, P, H, D):
    oc = of4.Cache(P, H, D, v_per_token=True)
    oc.write(k, v, slots)
    gc = f4.F4Cache(P, H, D, v_scale_per_token=True)
    f4.kv_cache_write_f4(gc, torch.from_numpy(np.ascontiguousarray(k)).cuda(),
                         torch.from_numpy(np.ascontiguousarray(v)).cuda(),
                         torch.from_numpy(np.asarray(slots, np.int32)).cuda())
    torch.cuda.synchronize()
    return gc, oc


@pytest.mark.parametrize("T,H,D,P", [(1, 1, 32, 1), (5, 2, 64, 2), (130, 4, 256, 4), (64 * 9 + 7, 4, 256, 12)])
def test_writer_bit_exact(T, H, D, P):
    g = synth.rng(700, T)
    k = synth.normal_f32(g, (T, H, D))
    v = synth.normal_f32(g, (T, H, D)) * np.float32(3.0)
    slots = g.permutation(P * 64)[:T].astype(np.int32)
    slots[::7] = -1
    gc, oc = _write_both(k, v, slots, P, H, D)
    assert tuple(gc.v_scale.shape) == (P, H, 64)
    assert cache_arrays_equal(gc, oc) == []


def test_writer_edge_rows_bit_exact():
    # zero rows, tiny and huge rows, a row scale of exactly 1 with values on and
    # one ulp around every half step, a single outlier deciding the row's scale
    g = synth.rng(701, 0)
    T, H, D = 64, 2, 256
    k = synth.normal_f32(g, (T, H, D))
    v = synth.normal_f32(g, (T, H, D))
    v[0, 0] = 0.0
    v[1, 0] *= np.float32(1e-6)
    v[2, 0] *= np.float32(1e-9)
    v[3, 0] = np.float32(7e5)
    v[3, 0, 5] = np.float32(-1e6)
    row = np.array([8.0] + [(j % 16 - 8) + 0.5 for j in range(255)], dtype=np.float32)
    v[4, 1] = row
    v[5, 1] = np.nextafter(row, np.float32(np.inf))
    v[6, 1] = np.nextafter(row, np.float32(-np.inf))
    v[7, 1, 200] = np.float32(300.0)
    gc, oc = _write_both(k, v, np.arange(T, dtype=np.int32), 1, H, D)
    assert cache_arrays_equal(gc, oc) == []


def _decode(ps, Hq, seed, W=1, wt=0, q_scale=1.0):
    bits, qv = random_q(len(ps.lengths), Hq, ps.D, seed, q_scale)
    out, m, l = f4.paged_attn_decode_f4(ps.gc, bf16_tensor(bits), ps.gpu_page_table(), ps.gpu_lengths(),
                                        max(ps.lengths), SM, num_windows=W, window_tokens=wt)
    torch.cuda.synchronize()
    ro, rm, rl = oracle_decode(ps, qv, SM, num_windows=W, window_tokens=wt)
    return (out.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()), (ro, rm, rl)


@pytest.mark.parametrize("lengths", [[1], [65], [130, 1, 700], [64 * 37 + 5]])
def test_decode_small_contexts(lengths):
    ps = PagedSet(lengths, Hkv=4, seed=710 + lengths[0], v_per_token=True)
    assert cache_arrays_equal(ps.gc, ps.oc) == []
    (o, m, l), (ro, rm, rl) = _decode(ps, 16, lengths[0])
    assert_attention_close(o, ro, f"lengths {lengths}")
    assert_states_close(m, l, rm, rl, f"lengths {lengths}")


@pytest.mark.parametrize("G,Hkv", [(1, 2), (2, 2), (8, 2)])
def test_decode_group_sizes(G, Hkv):
    ps = PagedSet([300, 1024], Hkv=Hkv, seed=720 + G, v_per_token=True)
    (o, m, l), (ro, rm, rl) = _decode(ps, G * Hkv, G)
    assert_attention_close(o, ro, f"G={G}")
    assert_states_close(m, l, rm, rl, f"G={G}")


def test_decode_windows_outliers_and_scaled_values():
    ps = PagedSet([3000, 130, 4096], Hkv=4, seed=730, outliers=True, v_scale=100.0, v_per_token=True)
    (o, m, l), (ro, rm, rl) = _decode(ps, 16, 730, W=5, wt=1024)
    assert_attention_close(o, ro, "windows")
    assert_states_close(m, l, rm, rl, "windows")
    out, M, L = f4.lse_merge(torch.from_numpy(m).cuda(), torch.from_numpy(l).cuda(), torch.from_numpy(o).cuda())
    (wo, _, _), _ = _decode(ps, 16, 730)
    assert_attention_close(out.cpu().numpy(), wo[0], "window fold")


@pytest.mark.parametrize("pos0,T", [(0, 64), (100, 37), (1000, 200)])
def test_prefill(pos0, T):
    ch = Chunk(pos0, T, seed=740 + pos0 + T, v_per_token=True)
    o, m, l = ch.run_gpu()
    ro, rm, rl = ch.run_oracle()
    assert cache_arrays_equal(ch.gc, ch.oc) == []
    assert_attention_close(o, ro, f"prefill pos0={pos0} T={T}")
    assert_states_close(m, l, rm, rl, f"prefill pos0={pos0} T={T}")


def test_decode_matches_the_per_block_layout_where_rows_share_a_scale():
    # rows whose 8 blocks have the same absmax quantise identically in both
    # layouts, so decode must give the same output over either cache
    g = synth.rng(750, 0)
    T, H, D = 500, 4, 256
    k = synth.normal_f32(g, (T, H, D))
    v = np.clip(synth.normal_f32(g, (T, H, D)), np.float32(-3.9), np.float32(3.9))
    v[:, :, ::32] = np.float32(4.0)  # every block's absmax is 4
    slots = np.arange(T, dtype=np.int32)
    P = (T + 63) // 64
    caches = []
    for vt in (False, True):
        c = f4.F4Cache(P, H, D, v_scale_per_token=vt)
        f4.kv_cache_write_f4(c, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(slots).cuda())
        caches.append(c)
    assert torch.equal(caches[0].v_nib, caches[1].v_nib)
    bits, _ = random_q(1, 16, D, 750)
    pt = torch.arange(P, dtype=torch.int32, device="cuda")[None]
    lens = torch.tensor([T], dtype=torch.int32, device="cuda")
    a = f4.paged_attn_decode_f4(caches[0], bf16_tensor(bits), pt, lens, T, SM)[0]
    b = f4.paged_attn_decode_f4(caches[1], bf16_tensor(bits), pt, lens, T, SM)[0]
    torch.cuda.synchronize()
    assert torch.allclose(a, b, rtol=0, atol=1e-6 * float(a.abs().max()))
