"""What the fp16 prefill's exact operand splits buy (test infrastructure, fp64).

The fp16 prefill feeds its matrix products exact pieces instead of single
fp16 roundings:
  * a dequantised key or value (n - 8) s is split as (n - 8) s_hi + (n - 8) s_lo
    with s_hi = the fp16 scale's top 8 significant bits (bits & 0xFFF8) and
    s_lo = s - s_hi; both products are exact in fp16;
  * a weight e (fp32) is split as hi = e rounded toward zero to fp16 and
    lo = (e - hi) rounded toward zero to fp16; e - hi is exact in fp32, and
    hi + lo misses e by less than 2^-20 of e (by less than fp16's subnormal
    step where lo is subnormal).
This module holds the arithmetic of those splits (`scale_split`, `rtz_fp16`)
and measures, against exact attention over the oracle's quantised cache,
what one plain fp16 rounding of the keys, the values or the weights would
cost instead (`single_rounding_errors`): the largest |error| of the output
over its RMS, the measure the parity tests bound by 2e-3.
"""
from __future__ import annotations

import numpy as np

import synth
from oracle import attention as oatt


def scale_split(s16: np.ndarray):
    """fp16 scales -> (s_hi, s_lo) as fp64: s_hi keeps the top 8 significant
    bits of the fp16 value, s_lo = s - s_hi (exact in fp64)."""
    bits = np.asarray(s16, dtype=np.float16).view(np.uint16)
    hi = (bits & np.uint16(0xFFF8)).view(np.float16).astype(np.float64)
    return hi, np.asarray(s16, dtype=np.float16).astype(np.float64) - hi


def rtz_fp16(x: np.ndarray) -> np.ndarray:
    """fp64 values (within fp16's finite range) rounded toward zero to fp16, as fp64."""
    x = np.asarray(x, dtype=np.float64)
    h = x.astype(np.float16)  # nearest even
    bits = h.view(np.uint16).copy()
    over = np.abs(h.astype(np.float64)) > np.abs(x)
    bits[over] -= np.uint16(1)  # one step toward zero (sign-magnitude encoding)
    return bits.view(np.float16).astype(np.float64)


def _fp16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def single_rounding_errors(n_keys=4096, rows=64, head_dim=256, sm_scale=1.0 / 16.0, outliers=True, seed=0):
    """max |out - exact| / RMS(exact) when only the keys, only the values or
    only the weights (P * 2^11, nearest even) are rounded once to fp16.
    K, V ~ N(0, 1) (with the synthetic outlier columns when `outliers`),
    quantised by the oracle's F4 writer; queries N(0, 1) rounded to bf16."""
    g = synth.rng(950 + seed, 0)
    K = synth.normal_f32(g, (n_keys, 1, head_dim))
    V = synth.normal_f32(g, (n_keys, 1, head_dim))
    q = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(synth.normal_f32(g, (rows, head_dim)))).astype(np.float64)
    if outliers:
        cols = synth.outlier_columns(g, 1, head_dim)
        synth.apply_outliers(K, cols)
        synth.apply_outliers(V, cols)
    Kd = oatt.dequantize_rows(K[:, 0])
    Vd = oatt.dequantize_rows(V[:, 0])

    def attend(Kx, Vx, round_p=None):
        s = (q @ Kx.T) * sm_scale
        p = np.exp(s - s.max(axis=1, keepdims=True))
        num = p if round_p is None else round_p(p * 2.0 ** 11) / 2.0 ** 11
        return (num @ Vx) / p.sum(axis=1, keepdims=True)

    exact = attend(Kd, Vd)
    rms = float(np.sqrt(np.mean(exact ** 2)))
    cases = {"K": attend(_fp16(Kd), Vd), "V": attend(Kd, _fp16(Vd)), "P": attend(Kd, Vd, _fp16)}
    return {k: float(np.abs(v - exact).max()) / rms for k, v in cases.items()}
