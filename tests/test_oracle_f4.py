"""Pins for the oracle's F4 quantiser and cache layout (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import f4

PINS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_pins.json")))
FMT = PINS["f4_format"]


def test_fp16_rounding_is_nearest_even_and_saturates():
    one = 1.0
    ulp = 2.0 ** -10
    r = f4.fp16_round(np.array([one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 2 ** -30,
                                65519.0, 65520.0, 1e9, 2.0 ** -25, 2.0 ** -25 + 2 ** -40]))
    assert r[0] == 1.0                      # tie -> even
    assert r[1] == 1.0 + 2 * ulp            # tie -> even (up)
    assert r[2] == 1.0 + ulp                # just past the tie -> up
    assert r[3] == 65504.0 and r[4] == 65504.0 and r[5] == 65504.0
    assert r[6] == 0.0                      # half the smallest subnormal: tie -> 0
    assert r[7] == 2.0 ** -24               # just above: smallest subnormal


def test_block_geometry_matches_pages():
    q = np.zeros((3, FMT["values_per_row"]), dtype=np.int8)
    assert f4.pack_block_bytes(q).shape == (3, FMT["bytes_per_row"])
    # a V row of head_dim values is head_dim/2 bytes of nibbles
    c = f4.Cache(1, 1, 256)
    assert c.v_nib[0, 0].size == 64 * 256 * FMT["v_row_bytes_per_head_dim"]
    assert c.k_nib[0, 0].size == 64 * 256 // 2


def test_zero_code_is_nibble_eight_and_nibble_order():
    q = np.zeros(32, dtype=np.int8)
    q[0], q[1], q[2], q[31] = -8, 7, 1, -1
    b = f4.pack_block_bytes(q)
    assert b[0] == (0 | (15 << 4))   # element 0 low nibble, element 1 high nibble
    assert b[1] == ((1 + 8) | (FMT["zero_code"] << 4))
    assert b[15] == (FMT["zero_code"] | (7 << 4))
    assert all(x == FMT["zero_code"] * 17 for x in b[2:15])
    assert np.array_equal(f4.unpack_block_bytes(b), q)


def test_values_are_nibble_minus_eight_times_scale():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((200, 32)).astype(np.float32)
    q, s = f4.quantize_blocks(x)
    nib = f4.unpack_block_bytes(f4.pack_block_bytes(q)).astype(np.int64) + 8
    assert nib.min() >= 0 and nib.max() <= 15
    xh = f4.dequantize_blocks(q, s)
    np.testing.assert_array_equal(xh, (nib - 8) * s.astype(np.float64)[:, None])


def test_grid_round_trip():
    # a block already on the grid (and holding code -8) re-quantises to itself
    rng = np.random.default_rng(4)
    s16 = rng.uniform(1e-3, 100, size=500).astype(np.float16)
    q = rng.integers(-8, 8, size=(500, 32)).astype(np.int8)
    q[:, 0] = -8
    x = (q.astype(np.float64) * s16.astype(np.float64)[:, None]).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), q * s16.astype(np.float64)[:, None])
    q2, s2 = f4.quantize_blocks(x)
    assert np.array_equal(s2, s16)
    assert np.array_equal(q2, q)


@pytest.mark.parametrize("dist", ["normal", "outlier", "tiny", "huge"])
def test_error_bound(dist):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4000, 32))
    if dist == "outlier":
        x[:, 3] *= 8
    elif dist == "tiny":
        x *= 1e-5
    elif dist == "huge":
        x *= 3e4
    x = x.astype(np.float32)
    q, s = f4.quantize_blocks(x)
    xd = x.astype(np.float64)
    sd = s.astype(np.float64)[:, None]
    err = np.abs(xd - f4.dequantize_blocks(q, s))
    a = np.abs(xd).max(axis=1, keepdims=True)
    clamped = xd > 7.5 * sd
    # the pages' bound max_abs/16 is half a step; fp16 rounding of the scale adds 2**-11
    assert np.all(err[~clamped] <= sd.repeat(32, 1)[~clamped] / 2)
    # for a normal fp16 scale that is max_abs/16 (1 + 2**-11); a subnormal scale
    # is rounded to an absolute 2**-25, adding at most 2**-26 to half a step
    bound = np.where(sd >= 2.0 ** -14, a / 16 * (1 + 2.0 ** -11), a / 16 + 2.0 ** -26)
    assert np.all(err[~clamped] <= bound.repeat(32, 1)[~clamped] * (1 + 1e-12))
    # only values above 7.5 steps clamp to code 7: error at most one step
    cb = np.where(sd >= 2.0 ** -14, sd * (1 + 2.0 ** -8), sd + 2.0 ** -22)
    assert np.all(err[clamped] <= cb.repeat(32, 1)[clamped])
    assert np.all(q[clamped] == 7)


def test_zero_block():
    q, s = f4.quantize_blocks(np.zeros((2, 32), dtype=np.float32))
    assert np.all(q == 0) and np.all(s == 0)
    assert np.all(f4.pack_block_bytes(q) == 0x88)


def test_power_of_two_scaling():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((300, 32)).astype(np.float32)
    q0, s0 = f4.quantize_blocks(x)
    for k in (-6, -1, 3, 9):
        q1, s1 = f4.quantize_blocks((x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1.astype(np.float64), s0.astype(np.float64) * 2.0 ** k)


def _exact_code(x: float, s: float) -> int:
    """The rule with rational arithmetic: nearest integer to x/s, ties to even, clamped."""
    if s == 0:
        return 0
    r = Fraction(x) / Fraction(s)
    fl = r.numerator // r.denominator
    rem = r - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return max(-8, min(7, fl))


def test_ties_and_near_ties_decided_exactly():
    # fp32 values within a few ulps of every half-step threshold, for scales
    # spanning many fp16 significands; compared against rational arithmetic
    rng = np.random.default_rng(7)
    scales = np.unique(rng.integers(0x0400, 0x7800, size=120).astype(np.uint16).view(np.float16))
    for s16 in scales:
        s = float(s16)
        xs = []
        for k in range(-8, 8):
            t = np.float32((k + 0.5) * s)
            u = t.view(np.uint32)
            for d in range(-3, 4):
                xs.append(np.uint32(int(u) + d).view(np.float32))
        xs = np.array(xs, dtype=np.float32)
        xs = xs[np.isfinite(xs) & (np.abs(xs.astype(np.float64)) <= 8 * s)]
        n = len(xs) // 32 * 32
        blk = xs[:n].reshape(-1, 32).copy()
        blk[:, 0] = np.float32(8 * s)  # force the block scale to s
        q, got_s = f4.quantize_blocks(blk)
        assert np.all(got_s == s16)
        for r in range(blk.shape[0]):
            for c in range(32):
                assert q[r, c] == _exact_code(float(blk[r, c]), s), (float(blk[r, c]), s)


def test_subnormal_scale():
    x = np.zeros(32, dtype=np.float32)
    x[5] = np.float32(3e-6)  # absmax/8 lies in fp16's subnormal range
    q, s = f4.quantize_blocks(x[None])
    assert 0 < float(s[0]) < 6.1e-5
    assert q[0, 5] == _exact_code(float(x[5]), float(s[0]))


def test_cache_layout_positions():
    # hand-derived from the layout spec: token 9 of page 2, kv head 1, D = 64
    c = f4.Cache(3, 2, 64)
    k = np.zeros((1, 2, 64), dtype=np.float32)
    v = np.zeros((1, 2, 64), dtype=np.float32)
    k[0, 1, 37] = 1.0        # block 1, element 5 -> byte 2 high nibble
    v[0, 1, 6] = -1.0        # dims 4..7 unit j = 1; dim 6 -> h = 1 low nibble
    c.write(k, v, np.array([2 * 64 + 9]))
    # K: code for 1.0 with s = 1/8 is 7 (clamped 8) -> nibble 15; others 8
    row = c.k_nib[2, 1, 1, 9]
    assert row[2] == (8 | (15 << 4))
    assert np.all(np.delete(row, 2) == 0x88)
    assert np.all(c.k_nib[2, 1, 0, 9] == 0x88)
    assert c.k_scale[2, 1, 9, 1] == np.float16(0.125) and c.k_scale[2, 1, 9, 0] == 0
    # V: token 9 -> unit c = 1, k = 0, r = 1 -> bytes 2 (h=0) and 3 (h=1) of unit j
    unit = c.v_nib[2, 1, 1, 1]
    assert unit[3] == (0 | (8 << 4))     # dim 6 code -8 -> nibble 0, dim 7 nibble 8
    assert unit[2] == 0x88
    assert np.all(unit[[0, 1]] == 0) and np.all(unit[4:] == 0)   # other tokens untouched
    assert np.all(c.v_nib[2, 1, 1, 0, 2:4] == 0x88)


def test_cache_round_trip_and_skip():
    rng = np.random.default_rng(8)
    P, H, D, T = 5, 2, 256, 40
    c = f4.Cache(P, H, D)
    k = rng.standard_normal((T, H, D)).astype(np.float32)
    v = rng.standard_normal((T, H, D)).astype(np.float32)
    slots = rng.permutation(P * 64)[:T]
    slots[3] = -1
    c.write(k, v, slots)
    kd = f4.dequantize_blocks(*f4.quantize_blocks(k.reshape(T, H, D // 32, 32))).reshape(T, H, D)
    vd = f4.dequantize_blocks(*f4.quantize_blocks(v.reshape(T, H, D // 32, 32))).reshape(T, H, D)
    for t in range(T):
        if slots[t] < 0:
            continue
        for h in range(H):
            a, b = c.page_values(slots[t] // 64, h)
            assert np.array_equal(a[slots[t] % 64], kd[t, h])
            assert np.array_equal(b[slots[t] % 64], vd[t, h])
    written = np.zeros(P * 64, bool)
    written[slots[slots >= 0]] = True
    for sl in np.nonzero(~written)[0][:20]:
        a, b = c.page_values(sl // 64, 0)
        assert np.all(a[sl % 64] == 0) and np.all(b[sl % 64] == 0)


# ---- per-token V scales (one scale per token per V head, mistral.rs PR #2375,
# "Changes by area" item 2) ---------------------------------------------------

def test_per_token_rows_follow_the_same_rule():
    # a whole 256-value row quantised as one group: scale from the row's absmax,
    # on-grid rows come back unchanged, zero rows give s = 0 / nibble 8, and the
    # error bound is half a step of the row's scale
    rng = np.random.default_rng(11)
    s16 = rng.uniform(1e-3, 100, size=64).astype(np.float16)
    q = rng.integers(-8, 8, size=(64, 256)).astype(np.int8)
    q[:, 17] = -8
    x = (q.astype(np.float64) * s16.astype(np.float64)[:, None]).astype(np.float32)
    q2, s2 = f4.quantize_group(x)
    assert np.array_equal(s2, s16) and np.array_equal(q2, q)
    z, sz = f4.quantize_group(np.zeros((3, 256), dtype=np.float32))
    assert np.all(z == 0) and np.all(sz == 0)
    y = (rng.standard_normal((500, 256)) * rng.uniform(1e-4, 1e3, (500, 1))).astype(np.float32)
    y[:, 9] *= 8  # an outlier channel sets the row's scale
    qy, sy = f4.quantize_group(y)
    yd = y.astype(np.float64)
    sd = sy.astype(np.float64)[:, None]
    assert np.array_equal(sy, f4.fp16_round(np.abs(yd).max(axis=1) * 0.125))
    err = np.abs(yd - f4.dequantize_blocks(qy, sy))
    clamped = yd > 7.5 * sd
    assert np.all(err[~clamped] <= np.broadcast_to(sd, err.shape)[~clamped] / 2)
    assert np.all(qy[clamped] == 7)
    # power-of-two scaling moves only the scale (scales kept inside fp16's normal range)
    w = rng.standard_normal((200, 256)).astype(np.float32)
    qw, sw = f4.quantize_group(w)
    for k in (-3, 5):
        qk, sk = f4.quantize_group((w * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(qk, qw) and np.array_equal(sk.astype(np.float64), sw.astype(np.float64) * 2.0 ** k)


def test_per_token_row_differs_from_cells_when_blocks_differ():
    # a row whose 32-value cells have different absmax: per-cell scales differ,
    # the per-token row has one scale (its absmax / 8) for all cells
    x = np.zeros((1, 256), dtype=np.float32)
    x[0, ::32] = np.arange(1, 9, dtype=np.float32)  # cell c has absmax c + 1
    qc, sc = f4.quantize_blocks(x.reshape(1, 8, 32))
    qr, sr = f4.quantize_group(x)
    assert np.array_equal(sc[0].astype(np.float64), np.arange(1, 9) / 8.0)
    assert float(sr[0]) == 1.0
    assert np.array_equal(qr[0, ::32], np.clip(np.arange(1, 9), -8, 7))
    assert np.array_equal(qc.reshape(1, 256)[0, ::32], np.full(8, 7))


def test_per_token_cache_layout_and_round_trip():
    rng = np.random.default_rng(12)
    P, H, D, T = 4, 2, 256, 50
    c = f4.Cache(P, H, D, v_per_token=True)
    assert c.v_scale.shape == (P, H, 64)
    # per token and head: 128 bytes of V nibbles and one 2-byte scale
    assert c.v_nib[0, 0].size // 64 + c.v_scale[0, 0].nbytes // 64 == 130
    k = rng.standard_normal((T, H, D)).astype(np.float32)
    v = rng.standard_normal((T, H, D)).astype(np.float32)
    v[:, :, 40] *= 8
    slots = rng.permutation(P * 64)[:T]
    slots[7] = -1
    c.write(k, v, slots)
    kd = f4.dequantize_blocks(*f4.quantize_blocks(k.reshape(T, H, D // 32, 32))).reshape(T, H, D)
    vq, vs = f4.quantize_group(v)
    vd = f4.dequantize_blocks(vq, vs)
    for t in range(T):
        if slots[t] < 0:
            continue
        for h in range(H):
            a, b = c.page_values(slots[t] // 64, h)
            assert np.array_equal(a[slots[t] % 64], kd[t, h])
            assert np.array_equal(b[slots[t] % 64], vd[t, h])
            assert c.v_scale[slots[t] // 64, h, slots[t] % 64] == vs[t, h]
    # the nibble bytes are laid out exactly as in the per-cell layout
    cb = f4.Cache(P, H, D)
    cb.put_codes(slots[slots >= 0] // 64, slots[slots >= 0] % 64, np.zeros_like(vq[slots >= 0]),
                 np.zeros((int((slots >= 0).sum()), H, D // 32), np.float16), vq[slots >= 0],
                 np.zeros((int((slots >= 0).sum()), H, D // 32), np.float16))
    assert np.array_equal(cb.v_nib, c.v_nib)


# ---- bf16 rounding and the gather of dequantised rows -------------------------

def test_bf16_round_ties_and_library_agreement():
    one = 1.0
    ulp = 2.0 ** -7  # bf16 keeps 8 significant bits
    r = f4.bf16_round(np.array([one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 2 ** -20, -(one + ulp / 2),
                                2.0 ** -130, 3.0 * 2 ** 100, 0.0]))
    assert r[0] == 1.0 and r[1] == 1.0 + 2 * ulp and r[2] == 1.0 + ulp and r[3] == -1.0
    assert r[4] == 2.0 ** -130 and r[5] == 3.0 * 2 ** 100 and r[6] == 0.0
    # against torch's own fp32 -> bf16 conversion (a library routine)
    import torch
    rng = np.random.default_rng(13)
    x = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-20, 20, 20000)).astype(np.float32)
    x[:64] = (np.arange(64) - 32 + 0.5) * np.float32(2.0 ** -3)  # exact ties at several magnitudes
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(f4.bf16_round(x.astype(np.float64)), ref)


@pytest.mark.parametrize("vt", [False, True])
def test_gather_rows_are_the_written_values(vt):
    rng = np.random.default_rng(14)
    P, H, D = 6, 2, 64
    lengths = [70, 0, 130]
    c = f4.Cache(P, H, D, v_per_token=vt)
    pt = np.full((3, 3), -1, np.int32)
    perm = rng.permutation(P)
    pt[0, :2] = perm[:2]
    pt[2, :3] = perm[2:5]
    rows_k, rows_v = [], []
    for b, n in enumerate(lengths):
        if n == 0:
            continue
        k = rng.standard_normal((n, H, D)).astype(np.float32)
        v = rng.standard_normal((n, H, D)).astype(np.float32)
        t = np.arange(n)
        c.write(k, v, pt[b, t // 64].astype(np.int64) * 64 + t % 64)
        rows_k.append(f4.dequantize_blocks(*f4.quantize_blocks(k.reshape(n, H, D // 32, 32))).reshape(n, H, D))
        rows_v.append(f4.dequantize_blocks(*f4.quantize_group(v)) if vt else
                      f4.dequantize_blocks(*f4.quantize_blocks(v.reshape(n, H, D // 32, 32))).reshape(n, H, D))
    K, V = c.gather(pt, lengths)
    assert np.array_equal(K, np.concatenate(rows_k)) and np.array_equal(V, np.concatenate(rows_v))
    # a page id outside the pool gives zero rows
    pt2 = pt.copy()
    pt2[2, 1] = P + 5
    K2, _ = c.gather(pt2, lengths)
    assert np.all(K2[70 + 64:70 + 128] == 0) and np.array_equal(K2[:70 + 64], K[:70 + 64])
