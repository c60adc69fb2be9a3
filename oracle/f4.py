"""F4 block quantiser and the paged cache's byte layout, fp64.  Test infrastructure only.

The format (mistral.rs PR #2375, "Changes by area" item 2): symmetric 4-bit
values stored as ``(nibble - 8) * scale``, 32 values per 16-byte row, one
scale per 32-value K cell.  For V the same item gives one scale per token per
V head; the default layout here gives V one fp16 scale per 32 contiguous
values like K (the workload description's granularity), and the per-token
variant (``v_per_token``) follows the page.  "Known limitations" on the same
page states the per-value error bound max_abs / 16.

Readings taken where the page is silent:
* scale s = fp16_round_nearest_even(absmax / 8), saturated to 65504; half a
  step is then absmax / 16, the page's bound;
* codes q = clamp(round_half_even(x / s), -8, 7) against the stored fp16 s,
  with the exact quotient; s == 0 gives all codes 0 (nibble 8);
* nibble = q + 8; byte m of a 32-value block holds elements 2m (low nibble)
  and 2m + 1 (high nibble).

Exactness of the quotient: x is fp32 and s is fp16, so if x / s is not
exactly k + 1/2 it differs from it by at least 2**-24 * |x / s| (the gap
between x and the exactly representable (k + 1/2) * s is at least one fp32
ulp of x).  A correctly rounded fp64 quotient errs by at most 2**-53 relative,
so fp64 division followed by round-half-even decides every case exactly.

Physical layout (one layer; P pages of 64 tokens, H kv heads, D = head_dim):
  k_nib   uint8  [P][H][D/32][64][16]   block c of token t: 16 bytes at (c, t)
  k_scale fp16   [P][H][64][D/32]
  v_nib   uint8  [P][H][8][D/4][16]     unit (c, j): tokens 8c..8c+7 x dims
                                        4j..4j+3; byte 4k + 2r + h holds dims
                                        4j+2h (low) and 4j+2h+1 (high) of token
                                        8c + 2k + r
  v_scale fp16   [P][H][64][D/32]        (per-token variant: [P][H][64])
"""
from __future__ import annotations

import numpy as np

PAGE = 64
BLOCK = 32
FP16_MAX = 65504.0


def fp16_round(a: np.ndarray) -> np.ndarray:
    """Round fp64 values to fp16, nearest-even, saturating at 65504."""
    a = np.minimum(np.asarray(a, dtype=np.float64), FP16_MAX)
    return a.astype(np.float16)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (8 significant bits, fp32's
    exponent range), ties to even; returned as fp64.  Finite inputs within
    bf16's range only."""
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros_like(a)
    nz = a != 0.0
    e = np.floor(np.log2(np.abs(a[nz])))
    # a power of two just below |a| can come out one too high from log2's rounding
    e = np.where(np.abs(a[nz]) < 2.0 ** e, e - 1, e)
    q = 2.0 ** (np.maximum(e, -126.0) - 7.0)  # spacing of bf16 values at that binade
    out[nz] = np.rint(a[nz] / q) * q          # exact scaling by a power of two; rint ties to even
    return out


def quantize_group(x: np.ndarray):
    """Quantise x[..., n] (fp32 values) with one scale per group along the last
    axis (n = 32 for a cell, head_dim for a per-token V row).  Returns (codes
    int8 in [-8, 7], scale fp16)."""
    x = np.asarray(x)
    xd = x.astype(np.float32).astype(np.float64)
    assert np.isfinite(xd).all(), "non-finite input to the F4 quantiser"
    a = np.abs(xd).max(axis=-1)
    s16 = fp16_round(a * 0.125)
    s = s16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0.0, np.rint(xd / np.where(s > 0.0, s, 1.0)), 0.0)
    q = np.clip(q, -8, 7).astype(np.int8)
    return q, s16


def quantize_blocks(x: np.ndarray):
    """Quantise x[..., 32] (fp32 values), one scale per 32-value cell."""
    assert np.shape(x)[-1] == BLOCK
    return quantize_group(x)


def dequantize_blocks(q: np.ndarray, s16: np.ndarray) -> np.ndarray:
    """(code) * scale with one scale per group along the last axis."""
    return q.astype(np.float64) * s16.astype(np.float64)[..., None]


def pack_block_bytes(q: np.ndarray) -> np.ndarray:
    """Codes [..., 32] -> bytes [..., 16]: element 2m low nibble, 2m + 1 high nibble."""
    n = (q.astype(np.int16) + 8).astype(np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def unpack_block_bytes(b: np.ndarray) -> np.ndarray:
    """Bytes [..., 16] -> codes [..., 32]."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (BLOCK,), dtype=np.int8)
    out[..., 0::2] = (b & 0x0F).astype(np.int8) - 8
    out[..., 1::2] = (b >> 4).astype(np.int8) - 8
    return out


class Cache:
    """The four arrays of one layer's paged F4 cache, in the physical layout above."""

    def __init__(self, num_pages: int, num_kv_heads: int, head_dim: int, v_per_token: bool = False):
        assert head_dim % BLOCK == 0
        P, H, D = num_pages, num_kv_heads, head_dim
        self.P, self.H, self.D = P, H, D
        self.v_per_token = bool(v_per_token)
        self.k_nib = np.zeros((P, H, D // BLOCK, PAGE, 16), dtype=np.uint8)
        self.v_nib = np.zeros((P, H, PAGE // 8, D // 4, 16), dtype=np.uint8)
        self.k_scale = np.zeros((P, H, PAGE, D // BLOCK), dtype=np.float16)
        vs_shape = (P, H, PAGE) if self.v_per_token else (P, H, PAGE, D // BLOCK)
        self.v_scale = np.zeros(vs_shape, dtype=np.float16)

    def put_codes(self, pages, offs, kq, ks, vq, vs):
        """Store codes kq, vq [N, H, D] and scales ks [N, H, D/32], vs [N, H, D/32]
        (per-token variant: [N, H]) at (page, offset) pairs."""
        pages = np.asarray(pages, dtype=np.int64)
        offs = np.asarray(offs, dtype=np.int64)
        N, H, D = kq.shape
        nb = D // BLOCK
        # K: 16 bytes per (block, token)
        kb = pack_block_bytes(kq.reshape(N, H, nb, BLOCK))          # [N, H, nb, 16]
        self.k_nib[pages[:, None, None], np.arange(H)[None, :, None],
                   np.arange(nb)[None, None, :], offs[:, None, None], :] = kb
        self.k_scale[pages, :, offs, :] = ks
        # V: for token t, dims 4j+2h, 4j+2h+1 go to byte 4k+2r+h of unit (t//8, j)
        n = (vq.astype(np.int16) + 8).astype(np.uint8).reshape(N, H, D // 4, 2, 2)
        vb = n[..., 0] | (n[..., 1] << 4)                               # [N, H, D/4, 2(h)]
        c = offs // 8
        base = 4 * ((offs % 8) // 2) + 2 * (offs % 2)
        for h in range(2):
            self.v_nib[pages[:, None, None], np.arange(H)[None, :, None], c[:, None, None],
                       np.arange(D // 4)[None, None, :], (base + h)[:, None, None]] = vb[..., h]
        self.v_scale[pages, :, offs] = vs

    def write(self, k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray):
        """Quantise k, v [T, H, D] (fp32) into the slots; slot -1 skips the token."""
        k = np.asarray(k, dtype=np.float32)
        v = np.asarray(v, dtype=np.float32)
        T, H, D = k.shape
        assert (H, D) == (self.H, self.D) and v.shape == k.shape
        slots = np.asarray(slot_mapping, dtype=np.int64)
        live = np.nonzero(slots >= 0)[0]
        assert len(np.unique(slots[live])) == len(live), "slot_mapping entries must be unique"
        if len(live) == 0:
            return
        nb = D // BLOCK
        kq, ks = quantize_blocks(k[live].reshape(len(live), H, nb, BLOCK))
        if self.v_per_token:
            vq, vs = quantize_group(v[live])  # one scale per (token, head) over all D values
        else:
            vq, vs = quantize_blocks(v[live].reshape(len(live), H, nb, BLOCK))
        self.put_codes(slots[live] // PAGE, slots[live] % PAGE,
                       kq.reshape(len(live), H, D), ks, vq.reshape(len(live), H, D), vs)

    def page_codes(self, page: int, head: int):
        """Codes [64, D] and fp16 scales [64, D/32] of K and V for one page-head
        tile (V scales [64] in the per-token variant)."""
        D, nb = self.D, self.D // BLOCK
        kb = self.k_nib[page, head]                                  # [nb, 64, 16]
        kc = unpack_block_bytes(kb).transpose(1, 0, 2).reshape(PAGE, D)
        u = self.v_nib[page, head]                                   # [8, D/4, 16]
        vc = np.empty((PAGE, D), dtype=np.int8)
        for t in range(PAGE):
            c, base = t // 8, 4 * ((t % 8) // 2) + 2 * (t % 2)
            for h in range(2):
                byte = u[c, :, base + h]
                vc[t, 2 * h::4] = (byte & 0x0F).astype(np.int8) - 8
                vc[t, 2 * h + 1::4] = (byte >> 4).astype(np.int8) - 8
        return kc, self.k_scale[page, head], vc, self.v_scale[page, head]

    def page_values(self, page: int, head: int):
        """Dequantised K and V of one page-head tile, fp64 [64, D] each."""
        kc, ks, vc, vs = self.page_codes(page, head)
        nb = self.D // BLOCK
        kd = dequantize_blocks(kc.reshape(PAGE, nb, BLOCK), ks).reshape(PAGE, self.D)
        if self.v_per_token:
            vd = dequantize_blocks(vc, vs)
        else:
            vd = dequantize_blocks(vc.reshape(PAGE, nb, BLOCK), vs).reshape(PAGE, self.D)
        return kd, vd

    def gather(self, page_table, lengths):
        """Dequantised K and V of each sequence's tokens, concatenated: fp64
        [sum(lengths), H, D] each (token i of sequence b at page_table[b][i // 64],
        slot i % 64; a page id outside the pool gives zero rows)."""
        page_table = np.asarray(page_table)
        total = int(sum(lengths))
        K = np.zeros((total, self.H, self.D))
        V = np.zeros((total, self.H, self.D))
        row = 0
        for b, n in enumerate(lengths):
            for lp in range((n + PAGE - 1) // PAGE):
                pid = int(page_table[b, lp])
                cnt = min(PAGE, n - lp * PAGE)
                if 0 <= pid < self.P:
                    for h in range(self.H):
                        kd, vd = self.page_values(pid, h)
                        K[row:row + cnt, h] = kd[:cnt]
                        V[row:row + cnt, h] = vd[:cnt]
                row += cnt
        return K, V

    def arrays(self):
        """The four arrays as raw bytes in C order (k_nib, k_scale bits, v_nib, v_scale bits)."""
        return (self.k_nib, self.k_scale.view(np.uint16), self.v_nib, self.v_scale.view(np.uint16))
