"""Static YaRN rope table and NEOX rotation, fp64.  Test infrastructure only.

Sources (the pages):
* mistral.rs PR #2375, "Changes by area" item 1: the table is resolved the way
  llama.cpp resolves it -- the attention factor nets to a table scale of
  ``1 + 0.1 ln(factor)`` (1.0199427025 at factor 1.220703125), and the
  interpolation ramp runs between correction dims derived from beta_fast = 32
  and beta_slow = 1, floored and ceiled as ggml does.
* ignis docs, context-and-speculation, ``--model-rope-scaling`` row: factor F
  in (1, 64]; the attention factor multiplies queries and keys alike, one
  table for every position ("static" YaRN, FreeToken issue #568, "What problem
  does this solve").
* mistral.rs PR #2375 item 1 names a partial rotary (``new_partial_yarn``) and
  an IMROPE-to-NEOX equivalence: rotation pairs are (i, i + rotary_dim/2) over
  the first ``rotary_dim`` channels; the rest pass through.

The pages print no formula.  The steps below are the published YaRN method
(frequency-dependent blend of interpolated and extrapolated frequencies, with
a linear ramp between two correction dimensions and a logarithmic attention
factor), written out in fp64.  Readings where the pages are silent:
* factor == 1 means plain RoPE with scale 1;
* ``mscale <= 0`` means "derive it": 1 + 0.1 ln(factor);
* the ramp denominator is guarded by 0.001 and the low/high dims are clamped to
  [0, rotary_dim - 1], the ggml convention the page points at.
"""
from __future__ import annotations

import math

import numpy as np


def base_inv_freq(theta: float, rotary_dim: int) -> np.ndarray:
    """theta_i = theta ** (-2 i / n) for pair index i < n/2."""
    n = int(rotary_dim)
    i = np.arange(n // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / n)


def correction_dim(rotary_dim: int, orig_ctx: int, beta: float, theta: float) -> float:
    """Real-valued pair index at which a frequency turns ``beta`` times over ``orig_ctx`` positions.

    Solving theta**(-2c/n) * L / (2 pi) = beta for c.
    """
    n = float(rotary_dim)
    return n * math.log(orig_ctx / (2.0 * math.pi * beta)) / (2.0 * math.log(theta))


def correction_range(rotary_dim: int, orig_ctx: int, beta_fast: float, beta_slow: float, theta: float):
    lo = math.floor(correction_dim(rotary_dim, orig_ctx, beta_fast, theta))
    hi = math.ceil(correction_dim(rotary_dim, orig_ctx, beta_slow, theta))
    return max(0, lo), min(rotary_dim - 1, hi)


def table_scale(factor: float, mscale: float = 0.0) -> float:
    """Attention factor folded into the table (scales queries and keys alike)."""
    if factor == 1.0:
        return 1.0 if mscale <= 0.0 else float(mscale)
    if mscale > 0.0:
        return float(mscale)
    return 1.0 + 0.1 * math.log(factor)


def yarn_inv_freq(theta: float, rotary_dim: int, factor: float, orig_ctx: int,
                  beta_fast: float, beta_slow: float) -> np.ndarray:
    """Blended per-pair frequency theta'_i.

    Pairs below the beta_fast correction dim keep theta_i (extrapolation),
    pairs above the beta_slow dim use theta_i / factor (interpolation), and a
    linear ramp mixes the two in between.
    """
    th = base_inv_freq(theta, rotary_dim)
    if factor == 1.0:
        return th
    lo, hi = correction_range(rotary_dim, orig_ctx, beta_fast, beta_slow, theta)
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    ramp = np.clip((i - lo) / max(0.001, hi - lo), 0.0, 1.0)
    keep = 1.0 - ramp  # weight of the extrapolated (unscaled) frequency
    return (th / factor) * (1.0 - keep) + th * keep


def yarn_table(params, positions):
    """cos and sin rows, each [N][rotary_dim/2], scaled by the table factor.

    ``params`` carries theta, rotary_dim, factor, orig_ctx, beta_fast,
    beta_slow, mscale (attribute access, e.g. ``synth.YarnSpec``).
    """
    f = yarn_inv_freq(params.theta, params.rotary_dim, params.factor, params.orig_ctx,
                      params.beta_fast, params.beta_slow)
    m = table_scale(params.factor, params.mscale)
    p = np.asarray(positions, dtype=np.float64).reshape(-1, 1)
    ang = p * f.reshape(1, -1)
    return m * np.cos(ang), m * np.sin(ang)


def rope_apply(x, cos, sin, rotary_dim: int):
    """NEOX rotation of the first ``rotary_dim`` channels of x[T, H, D].

    cos/sin are [T, rotary_dim/2]; channel i pairs with i + rotary_dim/2.
    Returns fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    h = rotary_dim // 2
    c = np.asarray(cos, dtype=np.float64)[:, None, :]
    s = np.asarray(sin, dtype=np.float64)[:, None, :]
    y = x.copy()
    a = x[..., :h]
    b = x[..., h:rotary_dim]
    y[..., :h] = a * c - b * s
    y[..., h:rotary_dim] = b * c + a * s
    return y
