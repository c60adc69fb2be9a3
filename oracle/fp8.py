"""The 8-bit prefill attention (Q.K^T in INT8, P.V in E4M3) as a model, fp64.  Test infrastructure only.

What is computed.  The ignis configuration page (context-and-speculation, the
``--model-prefill-attention`` row) offers an 8-bit precision for the prompt
attention's pass over a 4-bit-cache prefill chunk: the score product Q.K^T in
INT8 and the weighted sum P.V in E4M3, with an FP16 path as the fallback.  It
fixes neither the granularity of the scales nor the rounding.  The readings
below are this model's; each step is written out so that the GPU kernel can
be compared with it element by element, and the model itself is pinned
against the exact attention (``attention.prefill``) where every step is
exact and within its error budget elsewhere.

Readings (for one query row r at position p, head h, KV head g = h // (Hq/Hkv)):

1. Query to INT8, one power-of-two scale per row: e_r is the smallest integer
   with max_d |q_d| < 2^e_r, sigma_r = 2^(e_r - 7), Qi = clamp(rne(q / sigma_r),
   -127, 127) (round half to even; an all-zero row gives Qi = 0).
2. Cached keys to INT8, one power-of-two scale per token: with s_b the token's
   eight fp16 block scales, E_t = max(floor(log2 max_b s_b) + 1, -14) (the
   fp16 exponent field of the largest scale minus 14; -14 when every scale is
   zero or subnormal), tau_t = 2^(E_t - 4) and Kt = rne(c * s_b / tau_t) for
   the code c = nibble - 8 (to nearest, ties to even: the rule of the F4
   quantiser and of step 1).  |c * s_b / tau_t| < 128, so Kt lies in
   [-128, 112] without clamping.
3. Scores in log2 units: x = S * sigma_r * tau_t * qk, S = sum_d Qi_d Kt_d (an
   exact integer), qk = fp32(fp32(sm_scale) * fp32(log2 e)), the logit scale
   as the library forms it.
4. Keys t <= p are seen (causal over the cached prefix and the chunk itself).
5. Weights to E4M3 per group of 32 consecutive tokens (half a page): G = the
   smallest integer >= max x over the group's seen keys, P8 = e4m3(2^(x - G))
   (OCP E4M3, round to nearest even; subnormals kept); the group's weights
   carry the factor 2^G.
6. Values to E4M3 per page half and block of 32 channels: with E' the rule of
   step 2 applied to the V scales of the 32 cache slots of that page half and
   block (the single per-token scale when V has one scale per token),
   F = E' - 5 and V8 = e4m3(c * s / 2^F); |c * s / 2^F| < 256 < 448, so no value
   saturates.
7. out = sum_t P8 2^G V8 2^F / sum_t 2^x over the seen keys: the numerator
   takes the quantised weights, the denominator the unquantised ones.  The
   returned state is m = (max x) ln 2 and l = sum_t 2^(x - max x), the same
   convention as the exact prefill (natural-log max logit, sum of exp).

All arithmetic after the roundings above is exact or fp64; 2^x for the
denominator and 2^(x - G) before rounding are fp64.
"""
from __future__ import annotations

import math

import numpy as np

from .f4 import PAGE, BLOCK

LOG2E = 1.4426950408889634
E4M3_MAX = 448.0
GROUP = 32  # tokens per weight group (half a page)


# ---- E4M3 (OCP FP8 E4M3FN) --------------------------------------------------

def e4m3_value(code: int) -> float:
    """The value of an E4M3 byte: sign, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent field 0 holds the subnormals m * 2^-9; 0x7F / 0xFF are NaN."""
    code &= 0xFF
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    v = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def e4m3_round(x) -> np.ndarray:
    """Round fp64 values to the nearest E4M3 value, ties to even (the value
    whose last mantissa bit is 0).  |x| must not exceed 464 (the tie between
    448 and the first non-finite step, which rounds to 448)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    assert np.all(a <= 464.0), "value outside the E4M3 range"
    out = np.zeros_like(a)
    nz = a > 0.0
    # the spacing of E4M3 values at |x|: 2^(e - 3) in binade [2^e, 2^(e+1)), e >= -6; 2^-9 below 2^-6
    e = np.floor(np.log2(np.where(nz, a, 1.0)))
    e = np.where(np.where(nz, a, 1.0) < 2.0 ** e, e - 1, e)  # log2's rounding at powers of two
    q = 2.0 ** (np.maximum(e, -6.0) - 3.0)
    out[nz] = np.rint(a[nz] / q[nz]) * q[nz]  # rint: half to even; a / q is exact (power-of-two q)
    return np.where(x < 0, -out, out)


# ---- INT8 quantisers ---------------------------------------------------------

def _exp_bound(a: np.ndarray) -> np.ndarray:
    """Smallest integer e with a < 2^e, for a > 0 (elementwise)."""
    _, ex = np.frexp(a)  # a = f 2^ex, f in [0.5, 1)
    return ex.astype(np.int64)


def quantize_query_rows(q: np.ndarray):
    """Step 1: q [..., D] (exact values) -> (Qi int32 [..., D], sigma [...])."""
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q).max(axis=-1)
    e = np.where(a > 0, _exp_bound(np.where(a > 0, a, 1.0)), 7)
    sigma = np.ldexp(1.0, (e - 7).astype(np.int64))
    Qi = np.clip(np.rint(q / sigma[..., None]), -127, 127).astype(np.int32)
    return Qi, sigma


def scale_exponent(smax: np.ndarray) -> np.ndarray:
    """E = max(floor(log2 smax) + 1, -14), with -14 for smax == 0 (step 2)."""
    smax = np.asarray(smax, dtype=np.float64)
    e = np.where(smax > 0, _exp_bound(np.where(smax > 0, smax, 1.0)), -14)
    return np.maximum(e, -14).astype(np.int64)


def requantize_keys(codes: np.ndarray, scales: np.ndarray):
    """Step 2: codes c [N, D] (int), block scales s [N, D/32] (fp16 values) ->
    (Kt int32 [N, D], tau [N])."""
    s = np.asarray(scales, dtype=np.float64)
    E = scale_exponent(s.max(axis=-1))
    tau = np.ldexp(1.0, E - 4)
    sd = np.repeat(s, BLOCK, axis=-1)
    Kt = np.rint(codes.astype(np.float64) * sd / tau[:, None]).astype(np.int32)  # c s / tau is exact
    return Kt, tau


def logit_scale_log2(sm_scale: float) -> float:
    """qk of step 3: the fp32 product of the fp32 softmax scale and fp32 log2(e)."""
    return float(np.float32(np.float32(sm_scale) * np.float32(LOG2E)))


# ---- the model ----------------------------------------------------------------

def group_weights(x: np.ndarray):
    """Step 5 for groups of scores x [..., 32] (log2 units, -inf for keys not
    seen, at least one finite per group): (P8 [..., 32], G [...]) with
    G = ceil(max x) and P8 = e4m3(2^(x - G)): the largest weight before
    rounding lies in (1/2, 1]."""
    x = np.asarray(x, dtype=np.float64)
    G = np.ceil(x.max(axis=-1))
    return e4m3_round(np.exp2(x - G[..., None])), G


def _page_half_values(vc, vs, half: int):
    """V8 [32, D] and the factor 2^F [D] of one page half (step 6), from the
    page's value codes vc [64, D] and scales vs ([64, D/32], or [64])."""
    D = vc.shape[1]
    rows = slice(GROUP * half, GROUP * (half + 1))
    vc = vc[rows].astype(np.float64)
    vs = np.asarray(vs[rows], dtype=np.float64)
    if vs.ndim == 1:  # one V scale per token
        F = scale_exponent(vs.max()) - 5
        vals = vc * vs[:, None] * 2.0 ** (-F)
        f = np.full(D, 2.0 ** F)
    else:
        F = scale_exponent(vs.max(axis=0)) - 5       # per block
        sd = np.repeat(vs, BLOCK, axis=1)
        Fd = np.repeat(F, BLOCK)
        vals = vc * sd * np.ldexp(1.0, -Fd)[None, :]
        f = np.ldexp(1.0, Fd)
    return e4m3_round(vals), f


def prefill(cache, q, page_row, pos0: int, sm_scale: float, rows=None):
    """The 8-bit prefill of a chunk of T queries at positions pos0 .. pos0 + T - 1.

    The cache must already hold the chunk's own keys and values.  q: [T, Hq, D]
    (exact values, e.g. bf16).  ``rows`` optionally restricts the computed query
    indices (others stay 0).  Returns out [T, Hq, D], m [T, Hq], l [T, Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = cache.H
    Gq = Hq // Hkv
    rows = range(T) if rows is None else rows
    out = np.zeros((T, Hq, D))
    m = np.full((T, Hq), -np.inf)
    l = np.zeros((T, Hq))
    qk = logit_scale_log2(sm_scale)
    n_all = pos0 + T
    n_pages = (n_all + PAGE - 1) // PAGE
    Qi, sigma = quantize_query_rows(q)
    for g in range(Hkv):
        # keys and values of the sequence's pages, in logical token order
        Kt = np.zeros((n_pages * PAGE, D), dtype=np.int64)
        tau = np.zeros(n_pages * PAGE)
        V8 = np.zeros((n_pages * PAGE, D))
        Vf = np.zeros((n_pages * PAGE, D))
        for lp in range(n_pages):
            pg = int(page_row[lp])
            kc, ks, vc, vs = cache.page_codes(pg, g)
            kt, ta = requantize_keys(kc, ks)
            Kt[lp * PAGE:(lp + 1) * PAGE] = kt
            tau[lp * PAGE:(lp + 1) * PAGE] = ta
            for half in range(2):
                v8, f = _page_half_values(vc, vs, half)
                sl = slice(lp * PAGE + GROUP * half, lp * PAGE + GROUP * (half + 1))
                V8[sl] = v8
                Vf[sl] = f[None, :]
        Vd = V8 * Vf  # each quantised value times its group factor 2^F
        for i in rows:
            n = pos0 + i + 1
            for h in range(g * Gq, (g + 1) * Gq):
                S = Kt[:n] @ Qi[i, h].astype(np.int64)            # exact integers
                x = S.astype(np.float64) * sigma[i, h] * tau[:n] * qk
                M = x.max()
                ng = (n + GROUP - 1) // GROUP
                xg = np.full(ng * GROUP, -np.inf)
                xg[:n] = x                                  # groups of 32 keys, the last one padded
                p8, G = group_weights(xg.reshape(ng, GROUP))
                w = (p8 * np.exp2(G - M)[:, None]).reshape(-1)[:n]
                den = np.exp2(x - M).sum()
                out[i, h] = (w @ Vd[:n]) / den
                m[i, h] = M * math.log(2.0)
                l[i, h] = den
    return out, m, l
