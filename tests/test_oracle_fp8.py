"""Pins for the oracle's 8-bit prefill model (CPU only).

The E4M3 rounding is checked against an exhaustive nearest-value search over
the format's 254 finite codes (a different method from the oracle's binade
arithmetic) and the format's fixed points; the INT8 quantisers against their
error bounds, tie rules and the fp16 exponent field; the whole model against
the exact attention where every rounding step is exact, and against its
error budget elsewhere.
"""
import math

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import f4 as of4
from oracle import fp8

CODES = [c for c in range(256) if not math.isnan(fp8.e4m3_value(c))]
VALUES = np.array([fp8.e4m3_value(c) for c in CODES])


def nearest_code_value(x: float) -> float:
    """Brute force: the finite E4M3 value nearest x; on a tie the even code."""
    d = np.abs(VALUES - x)
    best = d.min()
    cands = [CODES[i] for i in np.nonzero(d == best)[0]]
    even = [c for c in cands if c % 2 == 0]
    c = even[0] if even else cands[0]
    return fp8.e4m3_value(c)


def test_e4m3_format_points():
    assert len(CODES) == 254
    assert fp8.e4m3_value(0x38) == 1.0                 # exponent bias 7
    assert fp8.e4m3_value(0x7E) == 448.0               # largest finite value
    assert fp8.e4m3_value(0x08) == 2.0 ** -6           # smallest normal
    assert fp8.e4m3_value(0x01) == 2.0 ** -9           # smallest subnormal
    assert fp8.e4m3_value(0x07) == 7 * 2.0 ** -9       # largest subnormal
    assert fp8.e4m3_value(0xB8) == -1.0
    # every finite value is a fixed point of the rounding
    np.testing.assert_array_equal(fp8.e4m3_round(VALUES), VALUES)


def test_e4m3_rounding_matches_exhaustive_search():
    g = np.random.default_rng(3)
    pos = np.sort(np.unique(np.abs(VALUES)))
    mids = (pos[:-1] + pos[1:]) / 2                     # every tie
    xs = np.concatenate([
        mids, -mids, mids * (1 + 2.0 ** -40), mids * (1 - 2.0 ** -40),
        np.exp(g.uniform(math.log(2.0 ** -12), math.log(448.0), 4000)) * g.choice([-1, 1], 4000),
        g.uniform(-1, 1, 500) * 2.0 ** -8,
    ])
    got = fp8.e4m3_round(xs)
    want = np.array([nearest_code_value(float(x)) for x in xs])
    np.testing.assert_array_equal(got, want)
    # ties go to the even mantissa: 1 + 1/16 -> 1, 1 + 3/16 -> 1.25, 1.5 * 2^-9 -> 2^-8, 2^-10 -> 0
    np.testing.assert_array_equal(fp8.e4m3_round([1.0625, 1.1875, 1.5 * 2.0 ** -9, 2.0 ** -10, 464.0]),
                                  [1.0, 1.25, 2.0 ** -8, 0.0, 448.0])


def test_query_rows_to_int8():
    g = np.random.default_rng(5)
    q = g.standard_normal((200, 256)) * np.exp(g.uniform(-6, 6, (200, 1)))
    q = of4.bf16_round(q)
    q[7] = 0.0
    Qi, sigma = fp8.quantize_query_rows(q)
    e = np.log2(sigma)
    assert np.all(e == np.round(e))                    # powers of two
    assert np.all(np.abs(Qi) <= 127)
    live = np.abs(q).max(axis=1) > 0
    mx = np.abs(Qi).max(axis=1)
    assert np.all(mx[live] >= 64) and mx[7] == 0       # the row's largest value uses the top bit
    err = np.abs(Qi * sigma[:, None] - q)
    clamped = np.abs(q / sigma[:, None]) > 127
    assert np.all(err[~clamped] <= sigma.repeat(256).reshape(err.shape)[~clamped] / 2)
    # half-way cases round to even: q / sigma = 2.5, 3.5, -2.5
    q2 = np.zeros((1, 256))
    q2[0, :4] = [100.0, 2.5, 3.5, -2.5]
    Qi2, s2 = fp8.quantize_query_rows(q2)
    assert s2[0] == 1.0 and list(Qi2[0, :4]) == [100, 2, 4, -2]
    # the clamp: 127.75 rounds to 128, kept at 127
    q2[0, 0] = 127.75
    assert fp8.quantize_query_rows(q2)[0][0, 0] == 127


def test_group_weights_put_the_largest_in_the_top_binade():
    g = np.random.default_rng(9)
    for _ in range(200):
        x = g.normal(0, 5, 32) + g.uniform(-100, 100)
        p8, G = fp8.group_weights(x)
        assert G == math.ceil(x.max()) and p8.shape == (32,)
        assert 0.5 <= p8.max() <= 1.0                 # 2^(x - G) in (1/2, 1], then rounded
        np.testing.assert_array_equal(p8, [nearest_code_value(v) for v in np.exp2(x - G)])
    # an integer maximum gives weight exactly 1; a score 10 below it rounds to 0 (below half of 2^-9);
    # groups are independent and unseen keys (-inf) weigh 0
    p8, G = fp8.group_weights(np.array([[3.0, 2.0, -7.0], [-0.5, -np.inf, -1.5]]))
    assert list(G) == [3, 0] and p8.tolist() == [[1.0, 0.5, 0.0], [fp8.e4m3_round(2 ** -0.5), 0.0,
                                                                     fp8.e4m3_round(2 ** -1.5)]]


def fp16_exponent_rule(smax):
    """E_t from the fp16 bit pattern: the exponent field of the largest scale minus 14."""
    bits = np.asarray(smax, dtype=np.float16).view(np.uint16).astype(np.int64)
    return ((bits >> 10) & 31) - 14


def test_scale_exponent_is_the_fp16_exponent_field():
    g = np.random.default_rng(6)
    bits = g.integers(0, 0x7C00, 5000).astype(np.uint16)     # every finite non-negative fp16
    s = bits.view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(fp8.scale_exponent(s), fp16_exponent_rule(s))
    assert fp8.scale_exponent(0.0) == -14


def test_keys_to_int8():
    g = np.random.default_rng(7)
    N = 3000
    codes = g.integers(-8, 8, (N, 256))
    scales = of4.fp16_round(np.exp(g.uniform(-12, 8, (N, 8)))).astype(np.float64)
    scales[:5] = 0.0
    scales[5] = 2.0 ** -20
    Kt, tau = fp8.requantize_keys(codes, scales)
    assert Kt.min() >= -128 and Kt.max() <= 112
    exact = codes * np.repeat(scales, 32, axis=1)
    assert np.all(np.abs(Kt * tau[:, None] - exact) <= tau[:, None] / 2)
    np.testing.assert_array_equal(np.log2(tau), fp16_exponent_rule(scales.max(axis=1)) - 4)
    # half-way cases round to the even integer
    c = np.zeros((1, 256), dtype=np.int64)
    c[0, :4] = [1, -1, 3, -3]
    s = np.zeros((1, 8))
    s[0, 0] = 1.5   # E = 1, tau = 2^-3: c * 1.5 / 2^-3 = 12 c (exact); use a second block to make ties
    s[0, 1] = 2.0 ** -4  # c * 2^-4 / 2^-3 = c / 2
    c[0, 32:36] = [1, -1, 3, -3]
    Kt, tau = fp8.requantize_keys(c, s)
    assert tau[0] == 2.0 ** -3
    assert list(Kt[0, :4]) == [12, -12, 36, -36]
    assert list(Kt[0, 32:36]) == [0, 0, 2, -2]          # 0.5 -> 0, -0.5 -> 0, 1.5 -> 2, -1.5 -> -2
    # ties toward every side: codes -8..7 over scale 2^-4 (c / 2): even neighbours only
    c2 = np.zeros((1, 256), dtype=np.int64)
    c2[0, 32:48] = np.arange(-8, 8)
    Kt2, _ = fp8.requantize_keys(c2, s)
    np.testing.assert_array_equal(Kt2[0, 32:48], [-4, -4, -3, -2, -2, -2, -1, 0, 0, 0, 1, 2, 2, 2, 3, 4])


def exact_case(seed, pos0, T, v_per_token=False):
    """A cache and queries for which every rounding of the model is exact.

    Each query row is one channel d0 at value 1 (Qi = 64, sigma = 2^-6); keys
    have power-of-two block scales within 2^3 of the token's largest, so the
    INT8 keys are exact, and the code of channel d0 lies in [-2, 7] with its
    block scale 4, so with qk = 1/4 every score is an integer in [-2, 7] and
    every weight 2^(x - G) >= 2^-9 is an E4M3 value.  Values have power-of-two
    scales, so every c s 2^-F is an E4M3 value.
    """
    g = np.random.default_rng(seed)
    H, D, Hq = 2, 256, 4
    n = pos0 + T
    npg = (n + 63) // 64
    P = npg + 1
    pt = g.permutation(P)[:npg].astype(np.int32)
    cache = of4.Cache(P, H, D, v_per_token=v_per_token)
    t = np.arange(n)
    pages, offs = pt[t // 64], t % 64
    kq = g.integers(-8, 8, (n, H, D)).astype(np.int8)
    d0s = g.integers(0, D, Hq)
    ks = np.ldexp(1.0, g.integers(-1, 3, (n, H, 8))).astype(np.float16)  # within 2^3 of each other
    for h in range(Hq):
        kv = h // (Hq // H)
        kq[:, kv, d0s[h]] = g.integers(-2, 8, n)
        ks[:, kv, d0s[h] // 32] = 4.0          # the largest scale, so 2^3 bound holds
    vq = g.integers(-8, 8, (n, H, D)).astype(np.int8)
    vs_shape = (n, H) if v_per_token else (n, H, 8)
    vs = np.ldexp(1.0, g.integers(-6, 1, vs_shape)).astype(np.float16)
    cache.put_codes(pages, offs, kq, ks, vq, vs)
    q = np.zeros((T, Hq, D))
    for h in range(Hq):
        q[:, h, d0s[h]] = 1.0
    # the fp32 softmax scale whose fp32 product with log2(e) is exactly 1/4
    sm = float(np.float32(0.25 / fp8.LOG2E))
    for _ in range(8):
        if fp8.logit_scale_log2(sm) == 0.25:
            break
        sm = float(np.nextafter(np.float32(sm), np.float32(1.0 if fp8.logit_scale_log2(sm) < 0.25 else 0.0)))
    assert fp8.logit_scale_log2(sm) == 0.25
    return cache, q, pt, sm


@pytest.mark.parametrize("seed,pos0,T,vtok", [(1, 0, 70, False), (2, 100, 40, False), (3, 37, 64, True)])
def test_model_equals_exact_attention_when_every_rounding_is_exact(seed, pos0, T, vtok):
    cache, q, pt, sm = exact_case(seed, pos0, T, vtok)
    o8, m8, l8 = fp8.prefill(cache, q, pt, pos0, sm)
    o, m, l = oatt.prefill(cache, q, pt, pos0, sm)
    # the exact oracle's logit scale is sm * log2(e) in fp64, the model's its fp32 product: ~1e-8 apart
    rms = np.sqrt(np.mean(o ** 2))
    assert np.abs(o8 - o).max() <= 1e-6 * rms
    np.testing.assert_allclose(m8, m, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(l8, l, rtol=1e-6)


def test_model_error_budget_on_random_inputs():
    """E4M3 keeps 3 mantissa bits: each weight and value is off by at most 2^-4
    relative, ~2^-4 / sqrt(3) RMS each; the INT8 scores add ~1%.  For
    independent errors the output's RMS error is about sqrt(2) * 3.6% + 1% of
    its RMS; the bound below allows 1.6 times that."""
    g = np.random.default_rng(11)
    H, D, Hq, pos0, T = 2, 256, 8, 300, 48
    n = pos0 + T
    npg = (n + 63) // 64
    pt = g.permutation(npg + 2)[:npg].astype(np.int32)
    cache = of4.Cache(npg + 2, H, D)
    t = np.arange(n)
    slots = (pt[t // 64].astype(np.int64) * 64 + t % 64).astype(np.int32)
    cache.write(g.standard_normal((n, H, D)).astype(np.float32), g.standard_normal((n, H, D)).astype(np.float32),
                slots)
    q = of4.bf16_round(g.standard_normal((T, Hq, D)))
    o8, m8, l8 = fp8.prefill(cache, q, pt, pos0, 1 / 16)
    o, m, l = oatt.prefill(cache, q, pt, pos0, 1 / 16)
    rms = np.sqrt(np.mean(o ** 2))
    err = o8 - o
    assert np.sqrt(np.mean(err ** 2)) <= 0.10 * rms
    assert np.abs(err).max() <= 0.6 * rms
    # the state: the max logit within the INT8 score error (~0.02 log2 units per
    # score); the total mass l e^m, which is what a fold uses, within ~1%
    assert np.abs(m8 - m).max() <= 0.05 * np.abs(m).max()
    assert np.abs((np.log(l8) + m8) - (np.log(l) + m)).max() <= 0.02


def test_model_within_the_error_predicted_from_the_formats():
    """The 8-bit model against the exact attention, each error divided by the
    standard deviation predicted from the formats' steps alone (tests/
    fp8_bound.py): RMS at most ~1 (the INT8 steps use upper bounds) and not
    vacuous, no value beyond 6.  Both V layouts, with outlier channels."""
    from fp8_bound import normalised_errors, predicted_sd
    g = np.random.default_rng(21)
    for vtok in (False, True):
        H, D, Hq, pos0, T = 2, 256, 8, 700, 40
        n = pos0 + T
        npg = (n + 63) // 64
        pt = g.permutation(npg + 2)[:npg].astype(np.int32)
        cache = of4.Cache(npg + 2, H, D, v_per_token=vtok)
        t = np.arange(n)
        slots = (pt[t // 64].astype(np.int64) * 64 + t % 64).astype(np.int32)
        k = g.standard_normal((n, H, D)).astype(np.float32)
        v = g.standard_normal((n, H, D)).astype(np.float32)
        k[:, :, [5, 77]] *= 8
        v[:, :, [5, 77]] *= 8
        cache.write(k, v, slots)
        q = of4.bf16_round(g.standard_normal((T, Hq, D)))
        o8, _, _ = fp8.prefill(cache, q, pt, pos0, 1 / 16)
        o, _, _ = oatt.prefill(cache, q, pt, pos0, 1 / 16)
        zs = []
        for kv in range(H):
            K, V = oatt.gather_values(cache, pt, n, kv)
            codes = [cache.page_codes(int(pt[lp]), kv) for lp in range(npg)]
            ks = np.concatenate([c[1] for c in codes])[:n].astype(np.float64)
            vs = np.concatenate([c[3] for c in codes])[:n].astype(np.float64)
            for i in range(0, T, 3):
                m = pos0 + i + 1
                hs = slice(kv * 4, kv * 4 + 4)
                sd = predicted_sd(q[i, hs], K[:m], V[:m], ks[:m], vs[:m], 1 / 16)
                zs.append(normalised_errors(o8[i, hs], o[i, hs], sd))
        z = np.concatenate([x.ravel() for x in zs])
        rms = math.sqrt(float(np.mean(z ** 2)))
        print(f"8-bit model vs exact: RMS of normalised error {rms:.3f}, max {np.abs(z).max():.2f}")
        assert 0.3 <= rms <= 1.2, rms
        assert np.abs(z).max() <= 6.0, np.abs(z).max()
