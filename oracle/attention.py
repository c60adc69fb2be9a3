"""Paged F4 attention by its plain definition, fp64.  Test infrastructure only.

What is computed (the pages' statement of the problem):
* grouped-query attention over 64-token pages (ignis context-and-speculation
  page, ``--model-adapt-context-step`` row: pages of 64 tokens), 4 KV heads of
  head_dim 256 serving 16 query heads (aeliusai "hybrid-attention-economics",
  table "What a token of context costs"); query head h reads KV head
  h // (Hq / Hkv);
* keys and values are the dequantised F4 cache (mistral.rs PR #2375,
  "Changes by area" item 2: the attention reads the packed cells and
  dequantises them, no dequantised copy is kept -- the oracle, by contrast,
  simply dequantises everything first);
* the softmax is exact: logits s_t = sm_scale * q . k_t, one max, one sum;
* a window of the context yields a partial state (m, l, o) -- the window's
  max logit, sum of exp(s - m), and normalised output -- and partial states
  fold by log-sum-exp (FreeToken issue #568, "Proposed solution" item 2:
  device windows folded by log2-sum-exp).  An empty window is (-inf, 0, 0);
* chunked prefill (ignis ``--model-prefill-chunk`` row; FreeToken #568 item 2
  device window): query i of a chunk at position pos0 + i attends causally to
  tokens [0, pos0 + i] of the cache after the chunk's own K/V were written.

The oracle splits work by pages only to bound memory; the arithmetic is one
exact max, one exact sum, in fp64, per output.
"""
from __future__ import annotations

import numpy as np

from .f4 import PAGE, BLOCK, dequantize_blocks, quantize_blocks

NEG_INF = float("-inf")


def gather_values(cache, page_row, n_tokens: int, head: int):
    """Dequantised K, V [n_tokens, D] of one sequence and KV head.

    Logical token t lives in physical page ``page_row[t // 64]``, slot t % 64.
    """
    D = cache.D
    K = np.empty((n_tokens, D), dtype=np.float64)
    V = np.empty((n_tokens, D), dtype=np.float64)
    for lp in range((n_tokens + PAGE - 1) // PAGE):
        kd, vd = cache.page_values(int(page_row[lp]), head)
        lo = lp * PAGE
        hi = min(n_tokens, lo + PAGE)
        K[lo:hi] = kd[:hi - lo]
        V[lo:hi] = vd[:hi - lo]
    return K, V


def partial_state(q, K, V, sm_scale: float):
    """(m, l, o) of one query row q[D] over keys K[n, D], values V[n, D]."""
    if K.shape[0] == 0:
        return NEG_INF, 0.0, np.zeros(V.shape[1], dtype=np.float64)
    s = sm_scale * (K @ np.asarray(q, dtype=np.float64))
    m = float(s.max())
    e = np.exp(s - m)
    l = float(e.sum())
    o = (e @ V) / l
    return m, l, o


def merge_states(ms, ls, os_):
    """Log-sum-exp fold of C partial states: m [C], l [C], o [C, D] -> (M, L, O)."""
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    os_ = np.asarray(os_, dtype=np.float64)
    live = ls > 0.0
    if not live.any():
        return NEG_INF, 0.0, np.zeros(os_.shape[-1], dtype=np.float64)
    M = ms[live].max()
    w = np.where(live, ls * np.exp(np.where(live, ms - M, 0.0)), 0.0)
    L = w.sum()
    O = (w[:, None] * os_).sum(axis=0) / L
    return float(M), float(L), O


def decode(cache, q, page_table, context_lens, sm_scale: float,
           window_tokens: int = 0, num_windows: int = 1):
    """Decode attention for B sequences.

    q: [B, Hq, D] (values, e.g. exact bf16); page_table [B, max_pages];
    context_lens [B].  With num_windows == 1 and window_tokens == 0 the window
    is the whole context.  Otherwise window w covers tokens
    [w * window_tokens, (w + 1) * window_tokens) of each sequence.
    Returns out [W, B, Hq, D], m [W, B, Hq], l [W, B, Hq] (W = num_windows).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = cache.H
    G = Hq // Hkv
    W = num_windows
    out = np.zeros((W, B, Hq, D))
    m = np.full((W, B, Hq), NEG_INF)
    l = np.zeros((W, B, Hq))
    for b in range(B):
        C = int(context_lens[b])
        for g in range(Hkv):
            K, V = gather_values(cache, page_table[b], C, g)
            for w in range(W):
                lo, hi = (0, C) if window_tokens == 0 else (w * window_tokens, min(C, (w + 1) * window_tokens))
                lo = min(lo, C)
                hi = max(hi, lo)
                for h in range(g * G, (g + 1) * G):
                    mm, ll, oo = partial_state(q[b, h], K[lo:hi], V[lo:hi], sm_scale)
                    out[w, b, h], m[w, b, h], l[w, b, h] = oo, mm, ll
    return out, m, l


def decode_rows(cache, q, page_table, context_lens, sm_scale: float,
                window_tokens: int = 0, num_windows: int = 1):
    """Decode of R query rows per sequence, as one round of speculative
    verification takes them (ignis context-and-speculation page,
    ``--spec-draft-tokens`` / ``--spec-draft-rows`` rows: a lane verifies up to
    7 drafted tokens, i.e. up to 8 rows, in one round).

    q: [B, R, Hq, D].  Row r of sequence b is the query at position
    C_b - R + r: it attends to tokens [0, C_b - R + r] (its own K/V, and those
    of the rows before it, are already in the cache), within each window as in
    ``decode``.  A row with no token (C_b - R + r < 0) gives (-inf, 0, 0).
    Returns out [W, B, R, Hq, D], m [W, B, R, Hq], l [W, B, R, Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    B, R, Hq, D = q.shape
    Hkv = cache.H
    G = Hq // Hkv
    W = num_windows
    out = np.zeros((W, B, R, Hq, D))
    m = np.full((W, B, R, Hq), NEG_INF)
    l = np.zeros((W, B, R, Hq))
    for b in range(B):
        C = int(context_lens[b])
        for g in range(Hkv):
            K, V = gather_values(cache, page_table[b], C, g)
            for r in range(R):
                n = max(0, C - R + r + 1)  # tokens this row sees
                for w in range(W):
                    lo, hi = (0, C) if window_tokens == 0 else (w * window_tokens, min(C, (w + 1) * window_tokens))
                    lo = min(lo, n)
                    hi = max(min(hi, n), lo)
                    for h in range(g * G, (g + 1) * G):
                        mm, ll, oo = partial_state(q[b, r, h], K[lo:hi], V[lo:hi], sm_scale)
                        out[w, b, r, h], m[w, b, r, h], l[w, b, r, h] = oo, mm, ll
    return out, m, l


def decode_head_from_values(q_rows, K, V, sm_scale: float, window_tokens: int = 0, num_windows: int = 1):
    """Decode for one KV head given its dequantised K, V [C, D] directly.

    q_rows [G, D].  Returns out [W, G, D], m [W, G], l [W, G].  Used where the
    cache is too large for the byte-level model: the values come from
    ``quantize_blocks``/``dequantize_blocks`` of the same fp32 inputs.  Logits
    are formed page chunk by page chunk purely to bound memory.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    C = K.shape[0]
    G = q_rows.shape[0]
    W = num_windows
    out = np.zeros((W, G, K.shape[1]))
    m = np.full((W, G), NEG_INF)
    l = np.zeros((W, G))
    for w in range(W):
        lo, hi = (0, C) if window_tokens == 0 else (w * window_tokens, min(C, (w + 1) * window_tokens))
        lo = min(lo, C)
        hi = max(hi, lo)
        if hi == lo:
            continue
        s = np.empty((G, hi - lo))
        step = 1 << 16
        for a in range(lo, hi, step):
            s[:, a - lo:min(hi, a + step) - lo] = sm_scale * (q_rows @ K[a:min(hi, a + step)].T)
        mm = s.max(axis=1)
        e = np.exp(s - mm[:, None])
        ll = e.sum(axis=1)
        acc = np.zeros((G, K.shape[1]))
        for a in range(lo, hi, step):
            acc += e[:, a - lo:min(hi, a + step) - lo] @ V[a:min(hi, a + step)]
        out[w] = acc / ll[:, None]
        m[w] = mm
        l[w] = ll
    return out, m, l


def dequantize_rows(x):
    """Quantise then dequantise fp32 rows x[..., D] (D a multiple of 32): the cache's values."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    q, s = quantize_blocks(x.reshape(*x.shape[:-1], D // BLOCK, BLOCK))
    return dequantize_blocks(q, s).reshape(x.shape)


def prefill(cache, q, page_row, pos0: int, sm_scale: float, rows=None):
    """Causal attention of a chunk of T queries at positions pos0 .. pos0 + T - 1.

    The cache must already hold the chunk's own keys and values.  q: [T, Hq, D].
    ``rows`` optionally restricts the computed query indices (others stay 0).
    Returns out [T, Hq, D], m [T, Hq], l [T, Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = cache.H
    G = Hq // Hkv
    rows = range(T) if rows is None else rows
    out = np.zeros((T, Hq, D))
    m = np.full((T, Hq), NEG_INF)
    l = np.zeros((T, Hq))
    n_all = pos0 + T
    for g in range(Hkv):
        K, V = gather_values(cache, page_row, n_all, g)
        for i in rows:
            n = pos0 + i + 1
            for h in range(g * G, (g + 1) * G):
                mm, ll, oo = partial_state(q[i, h], K[:n], V[:n], sm_scale)
                out[i, h], m[i, h], l[i, h] = oo, mm, ll
    return out, m, l
