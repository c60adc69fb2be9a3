"""paged_attn_decode_f4 and lse_merge on the GPU vs the oracle (max |delta| <= 2e-3 x output RMS)."""
import numpy as np
import pytest
import torch

import long_context_attention_kv_amd as f4
import synth
from oracle import attention as oatt
from gpu_cases import (PagedSet, assert_attention_close, assert_states_close, bf16_tensor, cache_arrays_equal,
                       oracle_decode, random_q)

pytestmark = pytest.mark.gpu
SM = 1.0 / 16.0


def _run(ps: PagedSet, Hq, seed=0, W=1, wt=0, q_scale=1.0, max_ctx=None, sm=SM):
    B = len(ps.lengths)
    bits, qv = random_q(B, Hq, ps.D, seed, q_scale)
    max_ctx = max(ps.lengths) if max_ctx is None else max_ctx
    out, m, l = f4.paged_attn_decode_f4(ps.gc, bf16_tensor(bits), ps.gpu_page_table(), ps.gpu_lengths(), max_ctx,
                                        sm, num_windows=W, window_tokens=wt)
    torch.cuda.synchronize()
    ro, rm, rl = oracle_decode(ps, qv, sm, num_windows=W, window_tokens=wt)
    return (out.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()), (ro, rm, rl)


@pytest.mark.parametrize("lengths", [[1], [63], [64], [65], [130, 1, 700], [64 * 37 + 5]])
def test_small_contexts(lengths):
    ps = PagedSet(lengths, Hkv=4, seed=len(lengths) * 100 + lengths[0])
    assert cache_arrays_equal(ps.gc, ps.oc) == []
    (o, m, l), (ro, rm, rl) = _run(ps, 16, seed=lengths[0])
    assert_attention_close(o, ro, f"lengths {lengths}")
    assert_states_close(m, l, rm, rl, f"lengths {lengths}")


@pytest.mark.parametrize("G,Hkv", [(1, 2), (2, 2), (4, 1), (8, 2)])
def test_group_sizes(G, Hkv):
    ps = PagedSet([300, 1024], Hkv=Hkv, seed=G)
    (o, m, l), (ro, rm, rl) = _run(ps, G * Hkv, seed=G)
    assert_attention_close(o, ro, f"G={G}")
    assert_states_close(m, l, rm, rl, f"G={G}")


def test_config0_shape():
    # one sequence of 4,096 tokens in a permuted pool of 64 pages, 16 query / 4 KV heads
    ps = PagedSet([4096], Hkv=4, seed=7, extra_pages=0)
    (o, m, l), (ro, rm, rl) = _run(ps, 16, seed=7)
    assert_attention_close(o, ro, "config0")
    assert_states_close(m, l, rm, rl, "config0")


def test_windows_and_empty_windows():
    ps = PagedSet([1000, 130, 4096], Hkv=4, seed=8)
    (o, m, l), (ro, rm, rl) = _run(ps, 16, seed=8, W=5, wt=1024)
    # windows past a sequence's end are the merge identity
    assert np.all(np.isneginf(m[1:, 0])) and np.all(l[1:, 0] == 0) and not o[1:, 0].any()
    assert_attention_close(o, ro, "windows")
    assert_states_close(m, l, rm, rl, "windows")
    # folding the windows on the GPU gives the whole-context answer
    out, M, L = f4.lse_merge(torch.from_numpy(m).cuda(), torch.from_numpy(l).cuda(), torch.from_numpy(o).cuda())
    (wo, wm, wl), _ = _run(ps, 16, seed=8)
    assert_attention_close(out.cpu().numpy(), wo[0], "window fold")


@pytest.mark.parametrize("B,W,wt", [(70, 1, 0), (90, 3, 256)])
def test_many_ranges_block_planner(B, W, wt):
    """More than 64 (window, sequence) ranges: the work list is built by the
    whole planning workgroup (W * B = 270 spans two batches of its 256 threads),
    with empty ranges (zero-length sequences, windows past a short sequence's
    end) among them."""
    print(f"decode: {B} sequences, {W} windows of {wt} tokens", flush=True)
    g = synth.rng(1300 + B, 0)
    lengths = [int(x) for x in g.integers(0, 900, B)]
    lengths[::11] = [0] * len(lengths[::11])
    lengths[5] = 64 * 12 + 3
    ps = PagedSet(lengths, Hkv=4, seed=1300 + B)
    (o, m, l), (ro, rm, rl) = _run(ps, 16, seed=B, W=W, wt=wt)
    for b, n in enumerate(lengths):
        for w in range(W):
            if n <= w * wt:  # outputs are [W, B, ...]
                assert np.all(np.isneginf(m[w, b])) and np.all(l[w, b] == 0) and not o[w, b].any()
    assert_attention_close(o, ro, f"{B} sequences, {W} windows")
    assert_states_close(m, l, rm, rl, f"{B} sequences, {W} windows")


def test_large_and_small_query_scale():
    ps = PagedSet([777], Hkv=4, seed=9)
    for sc in (1e-3, 30.0):
        (o, m, l), (ro, rm, rl) = _run(ps, 16, seed=9, q_scale=sc)
        assert_attention_close(o, ro, f"q scale {sc}")
        assert_states_close(m, l, rm, rl, f"q scale {sc}")


@pytest.mark.parametrize("offset", [3.0, -6.0])
def test_query_with_a_common_offset(offset):
    """Queries N(0, 1) + offset over outlier channels: the logits carry a large
    common term sum_c q_c (n_c - 8) s that an uncentred product (sum q n, then
    8 sum q taken off) would have to cancel."""
    print(f"decode, queries N(0,1) + {offset}", flush=True)
    ps = PagedSet([700, 130, 2000], Hkv=4, seed=31, outliers=True)
    g = synth.rng(231, 1)
    qf = synth.normal_f32(g, (3, 16, 256)) + np.float32(offset)
    bits = synth.f32_to_bf16_bits(qf)
    qv = synth.bf16_bits_to_f32(bits).astype(np.float64)
    out, m, l = f4.paged_attn_decode_f4(ps.gc, bf16_tensor(bits), ps.gpu_page_table(), ps.gpu_lengths(), 2000,
                                        SM / 4)
    torch.cuda.synchronize()
    ro, rm, rl = oracle_decode(ps, qv, SM / 4)
    rel = assert_attention_close(out.cpu().numpy(), ro, f"query offset {offset}")
    print(f"decode, queries N(0,1) + {offset}: max |delta| / RMS = {rel:.2e}", flush=True)
    assert_states_close(m.cpu().numpy(), l.cpu().numpy(), rm, rl, f"query offset {offset}")


@pytest.mark.parametrize("sm", [0.0, -1.0 / 16.0, 0.25])
def test_logit_scale_signs(sm):
    """A zero logit scale (uniform weights), a negative one and a large one."""
    ps = PagedSet([700, 90], Hkv=4, seed=12)
    (o, m, l), (ro, rm, rl) = _run(ps, 16, seed=12, sm=sm)
    assert_attention_close(o, ro, f"sm_scale {sm}")
    assert_states_close(m, l, rm, rl, f"sm_scale {sm}")


@pytest.mark.parametrize("log2_scale", [20, -30, -125])
def test_query_far_outside_fp16_range(log2_scale):
    """bf16 queries beyond fp16's largest value (x 2^20), below its smallest
    normal (x 2^-30) or at the bottom of bf16's own range (x 2^-125, partly
    subnormal); the logit scale compensates, so the weights stay the same."""
    ps = PagedSet([500], Hkv=4, seed=13)
    (o, m, l), (ro, rm, rl) = _run(ps, 16, seed=13, q_scale=2.0 ** log2_scale, sm=SM * 2.0 ** -log2_scale)
    assert_attention_close(o, ro, f"q x 2^{log2_scale}")
    assert_states_close(m, l, rm, rl, f"q x 2^{log2_scale}")


def test_tiny_query_gives_uniform_weights():
    """A query of bf16 values near 2^-125 with the plain logit scale: every
    logit is ~0, so the weights are uniform (the output is the mean value)."""
    ps = PagedSet([900, 130], Hkv=4, seed=14)
    (o, m, l), (ro, rm, rl) = _run(ps, 16, seed=14, q_scale=2.0 ** -125)
    assert_attention_close(o, ro, "tiny query")
    assert_states_close(m, l, rm, rl, "tiny query")


@pytest.mark.parametrize("sinks,mag", [([1234], 12.0), ([5], 30.0), ([77, 3000], 20.0), ([64, 65, 4000], 9.0)])
def test_dominant_tokens(sinks, mag):
    """Keys planted along the query of the group's first head (attention
    sinks), over N(0,1) keys and values with outlier channels and values x100:
    a few tokens carry most of the weight, so the output is close to their
    values and every rounding of those weights shows."""
    print(f"decode with dominant tokens {sinks}, logit {mag}", flush=True)
    lengths = [5000, 4100]
    bits, qv = random_q(2, 16, 256, seed=15)

    def plant(k):
        start = 0
        for b, n in enumerate(lengths):
            for g in range(4):
                d = qv[b, 4 * g] / np.linalg.norm(qv[b, 4 * g])
                for t in sinks:
                    # logit sm * q . k = mag for the group's first head
                    k[start + t, g] = (d * mag * 16.0 / np.linalg.norm(qv[b, 4 * g])).astype(np.float32)
            start += n

    ps = PagedSet(lengths, Hkv=4, seed=15, outliers=True, v_scale=100.0, k_edit=plant)
    out, m, l = f4.paged_attn_decode_f4(ps.gc, bf16_tensor(bits), ps.gpu_page_table(), ps.gpu_lengths(), 5000, SM)
    torch.cuda.synchronize()
    ro, rm, rl = oracle_decode(ps, qv, SM)
    o, m, l = out.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()
    assert_attention_close(o, ro, f"sinks {sinks}")
    assert_states_close(m, l, rm, rl, f"sinks {sinks}")


@pytest.mark.parametrize("seed", range(8))
def test_concentrated_attention_over_outlier_values(seed):
    """Short contexts (a few pages), outlier channels in K and V and queries
    x1.5: a handful of tokens hold most of the weight and the outputs of the
    outlier channels are many times the output RMS, the case that shows the
    rounding of the value weights most (in the tolerance's units)."""
    r = np.random.default_rng(4000 + seed)
    lengths = [int(x) for x in r.integers(8, 700, 3)]
    print(f"decode, concentrated attention: lengths {lengths}", flush=True)
    ps = PagedSet(lengths, Hkv=4, seed=400 + seed, outliers=True)
    bits, qv = random_q(3, 16, 256, seed=400 + seed, scale=1.5)
    out, m, l = f4.paged_attn_decode_f4(ps.gc, bf16_tensor(bits), ps.gpu_page_table(), ps.gpu_lengths(),
                                        max(lengths), SM)
    torch.cuda.synchronize()
    ro, rm, rl = oracle_decode(ps, qv, SM)
    rel = assert_attention_close(out.cpu().numpy(), ro, f"concentrated attention, lengths {lengths}")
    print(f"decode, concentrated attention: max |delta| / RMS = {rel:.2e}", flush=True)
    assert_states_close(m.cpu().numpy(), l.cpu().numpy(), rm, rl, "concentrated attention")


def test_outliers_and_scaled_values():
    ps = PagedSet([2000], Hkv=4, seed=10, outliers=True, v_scale=100.0)
    (o, m, l), (ro, rm, rl) = _run(ps, 16, seed=10)
    assert_attention_close(o, ro, "outliers")


def test_page_permutation_invariance_and_determinism():
    ps = PagedSet([3000, 64], Hkv=4, seed=11)
    bits, _ = random_q(2, 16, 256, 11)
    q = bf16_tensor(bits)
    a = f4.paged_attn_decode_f4(ps.gc, q, ps.gpu_page_table(), ps.gpu_lengths(), 3000, SM)[0]
    b = f4.paged_attn_decode_f4(ps.gc, q, ps.gpu_page_table(), ps.gpu_lengths(), 3000, SM)[0]
    assert torch.equal(a, b)
    # the same tokens in a different physical placement give the same result bit for bit
    ps2 = PagedSet([3000, 64], Hkv=4, seed=11, extra_pages=9, placement=5)
    c = f4.paged_attn_decode_f4(ps2.gc, q, ps2.gpu_page_table(), ps2.gpu_lengths(), 3000, SM)[0]
    assert torch.equal(a, c)


def test_context_lens_beyond_bound_are_clamped():
    ps = PagedSet([500], Hkv=4, seed=12)
    bits, qv = random_q(1, 16, 256, 12)
    lens = torch.tensor([10 ** 6], dtype=torch.int32, device="cuda")
    o, m, l = f4.paged_attn_decode_f4(ps.gc, bf16_tensor(bits), ps.gpu_page_table(), lens, 500, SM)
    ro, rm, rl = oracle_decode(ps, qv, SM)
    assert_attention_close(o.cpu().numpy(), ro, "clamped")


def test_zero_length_sequence():
    ps = PagedSet([0, 100], Hkv=4, seed=13)
    (o, m, l), (ro, rm, rl) = _run(ps, 16, seed=13)
    assert np.all(np.isneginf(m[0, 0])) and np.all(l[0, 0] == 0) and not o[0, 0].any()
    assert_attention_close(o, ro, "zero length")


@pytest.mark.parametrize("C,R", [(1, 3), (16, 16), (300, 5)])
def test_lse_merge_vs_oracle(C, R):
    g = synth.rng(500, C)
    m = (g.standard_normal((C, R)) * 5).astype(np.float32)
    l = g.uniform(0.5, 1000, (C, R)).astype(np.float32)
    o = g.standard_normal((C, R, 256)).astype(np.float32)
    m[0, 0] = -np.inf
    l[0, 0] = 0.0
    o[0, 0] = 0.0
    if R > 1:
        m[:, 1] = -np.inf
        l[:, 1] = 0.0
        o[:, 1] = 0.0
    out, M, L = f4.lse_merge(torch.from_numpy(m).cuda(), torch.from_numpy(l).cuda(), torch.from_numpy(o).cuda())
    out, M, L = out.cpu().numpy(), M.cpu().numpy(), L.cpu().numpy()
    for r in range(R):
        rm_, rl_, ro_ = oatt.merge_states(m[:, r], l[:, r], o[:, r])
        if rl_ == 0:
            assert np.isneginf(M[r]) and L[r] == 0 and not out[r].any()
            continue
        assert abs(M[r] - rm_) <= 1e-6 * max(1, abs(rm_))
        assert abs(L[r] - rl_) <= 1e-5 * rl_
        np.testing.assert_allclose(out[r], ro_, rtol=1e-5, atol=1e-5 * np.abs(ro_).max())


def test_kernel_timer_counts_decode_launches():
    ps = PagedSet([5000, 300], Hkv=4, seed=14)
    bits, _ = random_q(2, 16, 256, 14)
    q = bf16_tensor(bits)
    with f4.KernelTimer(f4.KERNEL_DECODE, max_launches=2) as t:
        for _ in range(3):  # the third launch is beyond max_launches
            f4.paged_attn_decode_f4(ps.gc, q, ps.gpu_page_table(), ps.gpu_lengths(), 5000, SM)
    assert t.launches == 2 and t.total_ms > 0.0
    with f4.KernelTimer(f4.KERNEL_PREFILL) as t2:  # a decode call is not a prefill launch
        f4.paged_attn_decode_f4(ps.gc, q, ps.gpu_page_table(), ps.gpu_lengths(), 5000, SM)
    assert t2.launches == 0
