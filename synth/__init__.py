"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This module only draws random numbers and arranges them into the shapes the
workloads use (page tables, context lengths, outlier columns, raw fp32/bf16
tensors).  It holds none of the attention, rope or quantisation arithmetic:
both the HIP path and the oracle receive what it returns and compute on their
own from there.

All draws come from numpy's PCG64 seeded through ``SeedSequence`` so that a
(config, layer, tensor) triple always yields the same values on any host.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

PAGE = 64
BASE_SEED = 20261203


def seed_seq(config: int, *path: int) -> np.random.SeedSequence:
    """Seed for one tensor: the config number plus a path such as (layer, tensor)."""
    return np.random.SeedSequence([BASE_SEED + int(config), *[int(p) for p in path]])


def rng(config: int, *path: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_seq(config, *path)))


def normal_f32(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(size=shape, dtype=np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the raw 16-bit patterns.

    This is the "cast to bf16" the workloads apply to their query draws; it is a
    storage conversion of the input, not part of the method.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def page_permutation(g: np.random.Generator, num_pages: int) -> np.ndarray:
    """A random placement of logical pages onto physical pages of one pool."""
    return g.permutation(num_pages).astype(np.int32)


def log_uniform_lengths(g: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths floor(exp(U(ln lo, ln hi)))."""
    u = g.uniform(math.log(lo), math.log(hi), size=n)
    return np.floor(np.exp(u)).astype(np.int64).clip(lo, hi).astype(np.int32)


def outlier_columns(g: np.random.Generator, num_kv_heads: int, head_dim: int, frac: float = 0.01) -> np.ndarray:
    """Indices of the (kv_head * head_dim + channel) columns scaled to mimic outlier channels."""
    total = num_kv_heads * head_dim
    k = int(round(frac * total))
    return np.sort(g.choice(total, size=k, replace=False)).astype(np.int64)


def apply_outliers(x: np.ndarray, cols: np.ndarray, factor: float = 8.0) -> np.ndarray:
    """Scale the chosen columns of x[..., Hkv, D] in place (viewed as [..., Hkv*D])."""
    shp = x.shape
    flat = x.reshape(*shp[:-2], shp[-2] * shp[-1])
    flat[..., cols] *= np.float32(factor)
    return x


def page_table_for(lengths, pool_perm: np.ndarray, max_pages: int) -> np.ndarray:
    """Hand out physical pages from one shared pool to sequences in order.

    Sequence b receives the next ceil(len_b / 64) entries of ``pool_perm``; unused
    table slots hold -1.
    """
    lengths = [int(x) for x in lengths]
    pt = np.full((len(lengths), max_pages), -1, dtype=np.int32)
    cur = 0
    for b, n in enumerate(lengths):
        npg = (n + PAGE - 1) // PAGE
        pt[b, :npg] = pool_perm[cur:cur + npg]
        cur += npg
    return pt


@dataclass
class YarnSpec:
    theta: float = 1.0e7
    rotary_dim: int = 256
    factor: float = 1.0
    orig_ctx: int = 262144
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    mscale: float = 0.0  # <= 0: derived from the factor


@dataclass
class DecodeWorkload:
    """Shape of one decode configuration (no data)."""
    name: str
    config: int
    lengths: list
    layers: int = 1
    num_q_heads: int = 16
    num_kv_heads: int = 4
    head_dim: int = 256
    yarn: YarnSpec = field(default_factory=YarnSpec)
    windows: int = 1
    window_tokens: int = 0
    outliers: bool = False


def decode_workloads():
    """The decode workloads, by config number."""
    y4 = YarnSpec(factor=4.0)
    return {
        0: DecodeWorkload("decode-1x4096", 0, [4096], yarn=YarnSpec(factor=1.0)),
        1: DecodeWorkload("decode-3x262144-16layers", 1, [262144] * 3, layers=16, yarn=y4, outliers=True),
        2: DecodeWorkload("decode-1x1048576-16windows", 2, [1048576], yarn=y4, windows=16, window_tokens=65536),
        4: DecodeWorkload("decode-ragged-8", 4, None, yarn=YarnSpec(factor=1.220703125)),
    }


def ragged_lengths(config: int = 4) -> list:
    return [int(x) for x in log_uniform_lengths(rng(config, 99), 8, 1024, 320000)]
