"""Pins for the oracle's YaRN table and rope rotation (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import yarn
from synth import YarnSpec

PINS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_pins.json")))


def test_table_scale_matches_printed_value():
    # mistral.rs PR #2375, "Changes by area" item 1: 1.0199427025 at factor 1.220703125
    p = PINS["yarn_table_scale"]
    m = yarn.table_scale(p["factor"])
    assert abs(m - p["table_scale"]) < 0.5e-10


def test_probe_factor_is_the_printed_context_ratio():
    p = PINS["yarn_probe_positions"]
    assert p["target_context"] / p["original_context"] == PINS["yarn_table_scale"]["factor"]


def test_plain_rope_when_factor_is_one():
    spec = YarnSpec(theta=1e7, rotary_dim=256, factor=1.0)
    pos = np.array([0, 1, 17, 4095, 1048575])
    c, s = yarn.yarn_table(spec, pos)
    # textbook RoPE: inverse frequencies 1 / theta^(2i/n), angle = position * inv_freq
    inv = 1.0 / (1e7 ** (np.arange(0, 256, 2, dtype=np.float64) / 256))
    ang = pos[:, None].astype(np.float64) * inv[None, :]
    # the two spellings of the frequency differ by an ulp, so the angle by ~ position * 1e-16
    tol = 1e-15 + 4e-16 * pos[:, None]
    assert np.all(np.abs(c - np.cos(ang)) <= tol)
    assert np.all(np.abs(s - np.sin(ang)) <= tol)


@pytest.mark.parametrize("rd", [256, 64])
@pytest.mark.parametrize("beta", [32.0, 1.0])
def test_correction_dim_turns_beta_times(rd, beta):
    # at the correction dim the frequency completes exactly beta turns over the original context
    L, th = 262144, 1e7
    c = yarn.correction_dim(rd, L, beta, th)
    freq = th ** (-2.0 * c / rd)
    assert abs(freq * L / (2 * math.pi) - beta) < 1e-9 * beta


@pytest.mark.parametrize("rd", [256, 64])
def test_correction_range_brackets_the_betas(rd):
    L, th = 262144, 1e7
    lo, hi = yarn.correction_range(rd, L, 32.0, 1.0, th)
    turns = lambda i: th ** (-2.0 * i / rd) * L / (2 * math.pi)
    # floor / ceil of the real dims: lo turns at least beta_fast times, lo+1 fewer;
    # hi turns at most beta_slow times, hi-1 more
    assert turns(lo) >= 32.0 > turns(lo + 1)
    assert turns(hi) <= 1.0 < turns(hi - 1)
    assert 0 <= lo < hi <= rd - 1


def _spec(factor, rd=256):
    return YarnSpec(theta=1e7, rotary_dim=rd, factor=factor, orig_ctx=262144, beta_fast=32, beta_slow=1)


@pytest.mark.parametrize("rd", [256, 64])
def test_low_pairs_keep_trained_frequency(rd):
    spec = _spec(4.0, rd)
    lo, hi = yarn.correction_range(rd, 262144, 32, 1, 1e7)
    m = yarn.table_scale(4.0)
    pos = np.array([1, 262143, 262144, 1048575])
    c, s = yarn.yarn_table(spec, pos)
    plain = _spec(1.0, rd)
    pc, ps = yarn.yarn_table(plain, pos)
    np.testing.assert_allclose(c[:, :lo + 1], m * pc[:, :lo + 1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(s[:, :lo + 1], m * ps[:, :lo + 1], rtol=0, atol=1e-12)


@pytest.mark.parametrize("rd", [256, 64])
def test_high_pairs_are_interpolated_by_the_factor(rd):
    # pairs at or above the slow correction dim run factor times slower:
    # the table at position 4k equals the plain table at position k (factor 4)
    spec = _spec(4.0, rd)
    lo, hi = yarn.correction_range(rd, 262144, 32, 1, 1e7)
    m = yarn.table_scale(4.0)
    k = np.array([1, 3, 65535, 262143])
    c, s = yarn.yarn_table(spec, 4 * k)
    pc, ps = yarn.yarn_table(_spec(1.0, rd), k)
    np.testing.assert_allclose(c[:, hi:], m * pc[:, hi:], rtol=0, atol=1e-9)
    np.testing.assert_allclose(s[:, hi:], m * ps[:, hi:], rtol=0, atol=1e-9)


def test_ramp_is_linear_between_the_correction_dims():
    rd, f = 256, 4.0
    lo, hi = yarn.correction_range(rd, 262144, 32, 1, 1e7)
    th = yarn.base_inv_freq(1e7, rd)
    tp = yarn.yarn_inv_freq(1e7, rd, f, 262144, 32, 1)
    # weight of the unscaled frequency in the blend
    w = (tp / th - 1.0 / f) / (1.0 - 1.0 / f)
    assert np.all(np.abs(w[:lo + 1] - 1.0) < 1e-12)
    assert np.all(np.abs(w[hi:]) < 1e-12)
    mid = w[lo:hi + 1]
    assert np.all(np.diff(mid) < 0)
    np.testing.assert_allclose(np.diff(mid, 2), 0.0, atol=1e-12)
    np.testing.assert_allclose(np.diff(mid), -1.0 / (hi - lo), atol=1e-12)


@pytest.mark.parametrize("factor", [1.0, 1.220703125, 4.0])
def test_position_zero_and_norm(factor):
    spec = _spec(factor)
    m = yarn.table_scale(factor)
    pos = np.array([0, 262144, 262145, 319999, 1048575])
    c, s = yarn.yarn_table(spec, pos)
    np.testing.assert_allclose(c[0], m, atol=0)
    np.testing.assert_allclose(s[0], 0.0, atol=0)
    np.testing.assert_allclose(c * c + s * s, m * m, rtol=1e-14)


def test_explicit_mscale_overrides():
    spec = YarnSpec(factor=4.0, mscale=1.5)
    c, s = yarn.yarn_table(spec, [0])
    assert c[0, 0] == 1.5


def test_probe_positions_high_precision():
    # fp64 evaluation vs a 50-digit evaluation of the same closed form at the
    # pages' probe positions.  fp64 carries the angle p * theta' to a few ulps,
    # so the bound scales with the angle (about 1e-11 at position 319,999).
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    f = PINS["yarn_table_scale"]["factor"]
    spec = _spec(f)
    pos = PINS["yarn_probe_positions"]["positions"] + [1048575]
    c, s = yarn.yarn_table(spec, pos)
    lo, hi = yarn.correction_range(256, 262144, 32, 1, 1e7)
    m = 1 + mpmath.mpf("0.1") * mpmath.log(mpmath.mpf(f))
    for i in [0, 5, lo, lo + 7, hi - 1, hi, 127]:
        th = mpmath.power(mpmath.mpf(10) ** 7, -mpmath.mpf(2 * i) / 256)
        r = min(1, max(0, mpmath.mpf(i - lo) / max(mpmath.mpf("0.001"), hi - lo)))
        tp = th / f * r + th * (1 - r)
        for j, p in enumerate(pos):
            tol = 1e-15 + 8e-16 * float(p * tp)
            assert abs(float(m * mpmath.cos(p * tp)) - c[j, i]) < tol
            assert abs(float(m * mpmath.sin(p * tp)) - s[j, i]) < tol


def test_rope_apply_is_complex_rotation():
    rng = np.random.default_rng(1)
    T, H, D, rd = 5, 3, 256, 256
    x = rng.standard_normal((T, H, D))
    pos = rng.integers(0, 1 << 20, size=T)
    c, s = yarn.yarn_table(_spec(4.0), pos)
    y = yarn.rope_apply(x, c, s, rd)
    z = (x[..., :rd // 2] + 1j * x[..., rd // 2:rd]) * (c + 1j * s)[:, None, :]
    np.testing.assert_allclose(y[..., :rd // 2], z.real, atol=1e-12)
    np.testing.assert_allclose(y[..., rd // 2:rd], z.imag, atol=1e-12)


def test_rope_apply_partial_passes_tail_and_composes():
    rng = np.random.default_rng(2)
    T, H, D, rd = 4, 2, 256, 64
    x = rng.standard_normal((T, H, D))
    p1 = rng.integers(0, 1 << 19, size=T)
    p2 = rng.integers(0, 1 << 19, size=T)
    sp = _spec(1.0, rd)
    c1, s1 = yarn.yarn_table(sp, p1)
    c2, s2 = yarn.yarn_table(sp, p2)
    c3, s3 = yarn.yarn_table(sp, p1 + p2)
    y = yarn.rope_apply(yarn.rope_apply(x, c1, s1, rd), c2, s2, rd)
    np.testing.assert_allclose(y, yarn.rope_apply(x, c3, s3, rd), atol=1e-9)
    assert np.array_equal(y[..., rd:], x[..., rd:])
    # the rotation keeps each pair's norm, times the table scale
    c, s = yarn.yarn_table(_spec(4.0, rd), p1)
    z = yarn.rope_apply(x, c, s, rd)
    m = yarn.table_scale(4.0)
    n0 = x[..., :rd // 2] ** 2 + x[..., rd // 2:rd] ** 2
    n1 = z[..., :rd // 2] ** 2 + z[..., rd // 2:rd] ** 2
    np.testing.assert_allclose(n1, m * m * n0, rtol=1e-12)
