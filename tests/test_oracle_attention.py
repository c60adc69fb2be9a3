"""Pins for the oracle's paged attention, partial states and their fold (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import f4

PAGE = 64


def _filled_cache(rng, n_pages, Hkv, D, lengths, perm=True, scale=1.0):
    """A cache holding random K/V for each sequence; returns (cache, page_table, fp32 K, V per seq)."""
    c = f4.Cache(n_pages, Hkv, D)
    pool = rng.permutation(n_pages) if perm else np.arange(n_pages)
    maxp = max((n + PAGE - 1) // PAGE for n in lengths)
    pt = np.full((len(lengths), maxp), -1, np.int32)
    cur = 0
    kv = []
    for b, n in enumerate(lengths):
        npg = (n + PAGE - 1) // PAGE
        pt[b, :npg] = pool[cur:cur + npg]
        cur += npg
        k = (scale * rng.standard_normal((n, Hkv, D))).astype(np.float32)
        v = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        t = np.arange(n)
        slots = pt[b, t // PAGE].astype(np.int64) * PAGE + t % PAGE
        c.write(k, v, slots)
        kv.append((k, v))
    return c, pt, kv


def _sdpa(q, K, V, sm_scale, causal_offset=None):
    """Textbook attention via torch in fp64: q [Hq, Lq, D], K/V [Hq, Lk, D]."""
    mask = None
    if causal_offset is not None:
        Lq, Lk = q.shape[1], K.shape[1]
        i = torch.arange(Lq)[:, None]
        j = torch.arange(Lk)[None, :]
        mask = j <= (causal_offset + i)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q), torch.as_tensor(K), torch.as_tensor(V), attn_mask=mask, scale=sm_scale).numpy()


@pytest.mark.parametrize("C", [1, 63, 64, 65, 130])
@pytest.mark.parametrize("G", [1, 4])
def test_decode_matches_textbook_attention(C, G):
    rng = np.random.default_rng(C * 10 + G)
    Hkv, D = 2, 64
    Hq = G * Hkv
    cache, pt, kv = _filled_cache(rng, 8, Hkv, D, [C, 70])
    q = rng.standard_normal((2, Hq, D))
    out, m, l = att.decode(cache, q, pt, [C, 70], 0.125)
    for b, n in enumerate([C, 70]):
        k, v = kv[b]
        Kd = att.dequantize_rows(k).transpose(1, 0, 2)  # [Hkv, n, D]
        Vd = att.dequantize_rows(v).transpose(1, 0, 2)
        # textbook GQA: each KV head serves G consecutive query heads
        Ke = np.repeat(Kd, G, axis=0)
        Ve = np.repeat(Vd, G, axis=0)
        ref = _sdpa(q[b][:, None, :], Ke, Ve, 0.125)[:, 0, :]
        np.testing.assert_allclose(out[0, b], ref, rtol=1e-12, atol=1e-12)
        s = 0.125 * np.einsum("hd,htd->ht", q[b], Ke)
        np.testing.assert_allclose(m[0, b], s.max(axis=1), rtol=1e-13)
        np.testing.assert_allclose(l[0, b], np.exp(s - s.max(axis=1, keepdims=True)).sum(axis=1), rtol=1e-12)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(11)
    cache, pt, kv = _filled_cache(rng, 4, 1, 256, [1])
    q = rng.standard_normal((1, 4, 256))
    out, m, l = att.decode(cache, q, pt, [1], 0.0625)
    vd = att.dequantize_rows(kv[0][1])[0, 0]
    for h in range(4):
        assert np.array_equal(out[0, 0, h], vd)
        assert l[0, 0, h] == 1.0


def test_uniform_logits_give_mean_value():
    rng = np.random.default_rng(12)
    cache, pt, kv = _filled_cache(rng, 6, 1, 64, [300])
    q = np.zeros((1, 4, 64))
    out, m, l = att.decode(cache, q, pt, [300], 0.125)
    vd = att.dequantize_rows(kv[0][1])[:, 0]
    np.testing.assert_allclose(out[0, 0, 0], vd.mean(axis=0), rtol=1e-12, atol=1e-14)
    assert m[0, 0, 0] == 0.0 and l[0, 0, 0] == 300.0


def test_dominant_logit_selects_its_value():
    rng = np.random.default_rng(13)
    D = 64
    c = f4.Cache(2, 1, D)
    k = np.zeros((100, 1, D), np.float32)
    v = rng.standard_normal((100, 1, D)).astype(np.float32)
    k[37, 0, :] = 1.0
    c.write(k, v, np.arange(100))
    pt = np.array([[0, 1]], np.int32)
    q = np.full((1, 1, D), 10.0)
    out, m, l = att.decode(c, q, pt, [100], 1.0)
    np.testing.assert_allclose(out[0, 0, 0], att.dequantize_rows(v)[37, 0], atol=1e-12)


def test_page_placement_does_not_matter():
    rng = np.random.default_rng(14)
    n, Hkv, D = 200, 2, 64
    k = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((1, 8, D))
    outs = []
    for perm in (np.arange(6), rng.permutation(6), rng.permutation(6)):
        c = f4.Cache(6, Hkv, D)
        pt = perm[None, :4].astype(np.int32)
        t = np.arange(n)
        c.write(k, v, pt[0, t // 64].astype(np.int64) * 64 + t % 64)
        outs.append(att.decode(c, q, pt, [n], 0.1)[0])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_merge_of_any_partition_equals_whole():
    rng = np.random.default_rng(15)
    n, D = 1000, 32
    K = rng.standard_normal((n, D)) * 2
    V = rng.standard_normal((n, D))
    q = rng.standard_normal(D)
    M, L, O = att.partial_state(q, K, V, 0.3)
    for _ in range(5):
        cuts = np.sort(rng.choice(np.arange(1, n), size=rng.integers(1, 12), replace=False))
        parts = np.split(np.arange(n), cuts)
        st = [att.partial_state(q, K[p], V[p], 0.3) for p in parts]
        m2, l2, o2 = att.merge_states([s[0] for s in st], [s[1] for s in st], [s[2] for s in st])
        assert abs(m2 - M) <= 1e-14 * abs(M)   # BLAS may order the dot products differently
        assert abs(l2 - L) <= 1e-12 * L
        np.testing.assert_allclose(o2, O, rtol=1e-12, atol=1e-13)


def test_merge_identity_and_associativity():
    rng = np.random.default_rng(16)
    D = 16
    e = att.partial_state(rng.standard_normal(D), np.zeros((0, D)), np.zeros((0, D)), 1.0)
    assert e[0] == float("-inf") and e[1] == 0.0 and not e[2].any()
    a = (1.5, 3.0, rng.standard_normal(D))
    b = (-2.0, 7.0, rng.standard_normal(D))
    c = (4.0, 0.5, rng.standard_normal(D))
    one = att.merge_states([a[0], e[0]], [a[1], e[1]], [a[2], e[2]])
    assert one[0] == a[0] and one[1] == a[1]
    np.testing.assert_allclose(one[2], a[2], rtol=1e-15, atol=0)
    ab = att.merge_states(*zip(a, b))
    left = att.merge_states(*zip(ab, c))
    bc = att.merge_states(*zip(b, c))
    right = att.merge_states(*zip(a, bc))
    np.testing.assert_allclose(left[2], right[2], rtol=1e-13)
    assert abs(left[1] - right[1]) <= 1e-13 * left[1]
    allempty = att.merge_states([e[0], e[0]], [0.0, 0.0], [e[2], e[2]])
    assert allempty[0] == float("-inf") and allempty[1] == 0.0


def test_windows_fold_to_whole_context():
    rng = np.random.default_rng(17)
    cache, pt, _ = _filled_cache(rng, 20, 2, 64, [1000, 130])
    q = rng.standard_normal((2, 8, 64))
    whole, wm, wl = att.decode(cache, q, pt, [1000, 130], 0.125)
    win, m, l = att.decode(cache, q, pt, [1000, 130], 0.125, window_tokens=256, num_windows=4)
    # sequence 1 has 130 tokens: windows 1..3 are empty (window 1 from 256 > 130)
    assert np.all(np.isneginf(m[1:, 1])) and np.all(l[1:, 1] == 0) and not win[1:, 1].any()
    for b in range(2):
        for h in range(8):
            M, L, O = att.merge_states(m[:, b, h], l[:, b, h], win[:, b, h])
            np.testing.assert_allclose(O, whole[0, b, h], rtol=1e-12, atol=1e-13)
            assert abs(M - wm[0, b, h]) <= 1e-14 * abs(M) and abs(L - wl[0, b, h]) <= 1e-12 * L


def test_values_path_equals_cache_path():
    rng = np.random.default_rng(18)
    n = 500
    cache, pt, kv = _filled_cache(rng, 10, 1, 256, [n])
    q = rng.standard_normal((1, 4, 256))
    a, am, al = att.decode(cache, q, pt, [n], 0.0625, window_tokens=128, num_windows=4)
    K = att.dequantize_rows(kv[0][0])[:, 0]
    V = att.dequantize_rows(kv[0][1])[:, 0]
    b, bm, bl = att.decode_head_from_values(q[0], K, V, 0.0625, window_tokens=128, num_windows=4)
    np.testing.assert_allclose(a[:, 0], b, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(am[:, 0], bm, rtol=1e-14)
    np.testing.assert_allclose(al[:, 0], bl, rtol=1e-12)


def test_prefill_causal_matches_textbook():
    rng = np.random.default_rng(19)
    Hkv, G, D, pos0, T = 2, 2, 64, 100, 37
    n = pos0 + T
    cache, pt, kv = _filled_cache(rng, 4, Hkv, D, [n])
    q = rng.standard_normal((T, G * Hkv, D))
    out, m, l = att.prefill(cache, q, pt[0], pos0, 0.2)
    Kd = np.repeat(att.dequantize_rows(kv[0][0]).transpose(1, 0, 2), G, axis=0)
    Vd = np.repeat(att.dequantize_rows(kv[0][1]).transpose(1, 0, 2), G, axis=0)
    ref = _sdpa(q.transpose(1, 0, 2), Kd, Vd, 0.2, causal_offset=pos0)
    np.testing.assert_allclose(out, ref.transpose(1, 0, 2), rtol=1e-12, atol=1e-12)
    # the last row is a decode at position pos0 + T - 1
    dec, _, _ = att.decode(cache, q[-1][None], pt, [n], 0.2)
    np.testing.assert_allclose(out[-1], dec[0, 0], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("C", [1, 65, 130])
def test_decode_over_per_token_v_scales_matches_textbook_attention(C):
    # the same definition over a cache whose V rows carry one scale per token
    rng = np.random.default_rng(900 + C)
    Hkv, D, G = 2, 64, 4
    c = f4.Cache(4, Hkv, D, v_per_token=True)
    pt = np.full((1, 3), -1, np.int32)
    npg = (C + PAGE - 1) // PAGE
    pt[0, :npg] = rng.permutation(4)[:npg]
    k = rng.standard_normal((C, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((C, Hkv, D)).astype(np.float32)
    v[:, :, 5] *= 8
    t = np.arange(C)
    c.write(k, v, pt[0, t // PAGE].astype(np.int64) * PAGE + t % PAGE)
    q = rng.standard_normal((1, G * Hkv, D))
    out, m, l = att.decode(c, q, pt, [C], 0.125)
    Kd = att.dequantize_rows(k).transpose(1, 0, 2)
    vq, vs = f4.quantize_group(v)
    Vd = f4.dequantize_blocks(vq, vs).transpose(1, 0, 2)
    ref = _sdpa(q[0][:, None, :], np.repeat(Kd, G, axis=0), np.repeat(Vd, G, axis=0), 0.125)[:, 0]
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-12, atol=1e-12)
    if C == 1:  # one token: the output is that token's dequantised V row
        np.testing.assert_array_equal(out[0, 0], np.repeat(Vd[:, 0], G, axis=0))


# ---- several query rows per sequence (speculative verification rounds) -------

def test_decode_rows_single_row_is_decode_and_rows_are_prefill_rows():
    rng = np.random.default_rng(950)
    Hkv, D, G, R = 2, 64, 2, 3
    lengths = [130, 2, 64]
    cache, pt, kv = _filled_cache(rng, 12, Hkv, D, lengths)
    q = rng.standard_normal((3, R, G * Hkv, D))
    out, m, l = att.decode_rows(cache, q, pt, lengths, 0.125)
    # one row per sequence is plain decode
    o1, m1, l1 = att.decode_rows(cache, q[:, -1:], pt, lengths, 0.125)
    d, dm, dl = att.decode(cache, q[:, -1], pt, lengths, 0.125)
    np.testing.assert_array_equal(o1[:, :, 0], d)
    np.testing.assert_array_equal(m1[:, :, 0], dm)
    # row r equals a decode over the first C - R + r + 1 tokens
    for r in range(R):
        lens_r = [max(0, n - R + r + 1) for n in lengths]
        dr, dmr, dlr = att.decode(cache, q[:, r], pt, lens_r, 0.125)
        np.testing.assert_allclose(out[:, :, r], dr, rtol=1e-13, atol=1e-13)
        np.testing.assert_array_equal(m[:, :, r], dmr)
    # the sequence of 2 tokens: its first row (position -1) sees nothing
    assert np.isneginf(m[0, 1, 0]).all() and (l[0, 1, 0] == 0).all() and not out[0, 1, 0].any()
    # and the R rows of a sequence are the prefill rows of a chunk at C - R
    for b, n in enumerate(lengths):
        if n < R:
            continue
        po, pm, pl = att.prefill(cache, q[b], pt[b], n - R, 0.125)
        np.testing.assert_allclose(out[0, b], po, rtol=1e-13, atol=1e-13)


def test_decode_rows_windows_fold_to_the_whole_context():
    rng = np.random.default_rng(951)
    Hkv, D, G, R = 1, 64, 4, 4
    lengths = [300]
    cache, pt, kv = _filled_cache(rng, 6, Hkv, D, lengths)
    q = rng.standard_normal((1, R, G, D))
    ow, mw, lw = att.decode_rows(cache, q, pt, lengths, 0.125, window_tokens=128, num_windows=3)
    o, m, l = att.decode_rows(cache, q, pt, lengths, 0.125)
    for r in range(R):
        for h in range(G):
            M, L, O = att.merge_states(mw[:, 0, r, h], lw[:, 0, r, h], ow[:, 0, r, h])
            np.testing.assert_allclose(O, o[0, 0, r, h], rtol=1e-12, atol=1e-12)
            assert abs(M - m[0, 0, r, h]) <= 1e-12 and abs(L - l[0, 0, r, h]) <= 1e-9 * L
