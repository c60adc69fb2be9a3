"""Out-of-range page ids in a page table: the kernels drop that page's tokens
(they cannot be checked on the host; the library's contract is to skip them
rather than read outside the pool).  The expected result is the attention over
the remaining tokens, from the oracle."""
import numpy as np
import pytest
import torch

import long_context_attention_kv_amd as f4
from oracle import attention as oatt
from oracle import fp8 as ofp8
from gpu_cases import (PagedSet, assert_attention_close, assert_states_close, bf16_tensor, bf16_values,
                       random_q)
from test_gpu_prefill import Chunk, PAGE, SM

pytestmark = pytest.mark.gpu


def test_decode_drops_out_of_range_pages():
    print("decode with out-of-range page ids", flush=True)
    ps = PagedSet([700, 300], seed=31)
    pt = ps.pt.copy()
    dropped = {0: [2, 7], 1: [1]}
    pt[0, 2] = ps.num_pages + 5   # past the pool
    pt[0, 7] = -1
    pt[1, 1] = -7
    bits, qv = random_q(2, 16, 256, seed=31)
    out, m, l = f4.paged_attn_decode_f4(ps.gc, bf16_tensor(bits), torch.from_numpy(pt).cuda(), ps.gpu_lengths(),
                                        700, SM)
    torch.cuda.synchronize()
    out, m, l = out.cpu().numpy()[0], m.cpu().numpy()[0], l.cpu().numpy()[0]
    for b, n in enumerate(ps.lengths):
        keep = np.ones(n, bool)
        for lp in dropped[b]:
            keep[lp * PAGE:(lp + 1) * PAGE] = False
        for g in range(4):
            K, V = oatt.gather_values(ps.oc, ps.pt[b], n, g)
            ro, rm, rl = oatt.decode_head_from_values(qv[b, 4 * g:4 * g + 4], K[keep], V[keep], SM)
            assert_attention_close(out[b, 4 * g:4 * g + 4], ro[0], f"decode b={b} kv head {g}")
            assert_states_close(m[b, 4 * g:4 * g + 4], l[b, 4 * g:4 * g + 4], rm[0], rl[0], f"decode b={b} g={g}")


def chunk_with_a_dropped_prefix_page():
    ch = Chunk(300, 70, seed=880)
    pt_gpu = ch.pt.copy()
    pt_gpu[1] = ch.P + 11          # logical page 1 (tokens 64..127 of the prefix) points past the pool
    t = np.arange(ch.pos0, ch.pos0 + ch.T)
    slots = (ch.pt[t // PAGE].astype(np.int64) * PAGE + t % PAGE).astype(np.int32)
    ch.oc.write(ch.k_new, ch.v_new, slots)
    return ch, pt_gpu


@pytest.mark.parametrize("fp8", [False, True])
def test_prefill_drops_out_of_range_pages(fp8):
    print(f"prefill ({'8-bit' if fp8 else 'fp16'}) with an out-of-range page id", flush=True)
    ch, pt_gpu = chunk_with_a_dropped_prefix_page()
    fn = f4.paged_attn_prefill_f4_fp8 if fp8 else f4.paged_attn_prefill_f4
    o, m, l = fn(ch.gc, bf16_tensor(ch.qbits), torch.from_numpy(ch.k_new).cuda(), torch.from_numpy(ch.v_new).cuda(),
                 torch.from_numpy(pt_gpu).cuda(), ch.pos0, SM)
    torch.cuda.synchronize()
    o, m, l = o.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()
    qv = bf16_values(ch.qbits)
    if fp8:
        # dropping a whole page keeps the 32-token groups of the others and the
        # causal order, so the model over the table without it (positions shifted
        # by one page) is the expected result
        page_row = np.delete(ch.pt, 1)
        ro, rm, rl = ofp8.prefill(ch.oc, qv, page_row, ch.pos0 - PAGE, SM)
        assert_attention_close(o, ro, "8-bit prefill, page 1 dropped")
        assert_states_close(m, l, rm, rl, "8-bit prefill, page 1 dropped")
        return
    n_all = ch.pos0 + ch.T
    for g in range(4):
        K, V = oatt.gather_values(ch.oc, ch.pt, n_all, g)
        keep = np.ones(n_all, bool)
        keep[PAGE:2 * PAGE] = False
        for i in range(0, ch.T, 7):
            n = ch.pos0 + i + 1
            ro, rm, rl = oatt.decode_head_from_values(qv[i, 4 * g:4 * g + 4], K[:n][keep[:n]], V[:n][keep[:n]], SM)
            assert_attention_close(o[i, 4 * g:4 * g + 4], ro[0], f"prefill row {i} kv head {g}")
            assert_states_close(m[i, 4 * g:4 * g + 4], l[i, 4 * g:4 * g + 4], rm[0], rl[0], f"prefill row {i} g={g}")


@pytest.mark.parametrize("fp8", [False, True])
def test_prefill_write_skips_huge_page_ids(fp8):
    """The chunk's own pages carry ids 2^26 and 2^26 + 1: the in-call write must
    leave every cell of the pool unchanged (an id times 64 overflows int32 and
    would wrap onto a live page), and the attention drops those pages."""
    print(f"prefill ({'8-bit' if fp8 else 'fp16'}) writing through page ids 2^26, 2^26 + 1", flush=True)
    ch = Chunk(128, 128, seed=881)
    pt_gpu = ch.pt.copy()
    pt_gpu[2] = 1 << 26
    pt_gpu[3] = (1 << 26) + 1
    before = [t.clone() for t in (ch.gc.k_nib, ch.gc.k_scale, ch.gc.v_nib, ch.gc.v_scale)]
    fn = f4.paged_attn_prefill_f4_fp8 if fp8 else f4.paged_attn_prefill_f4
    o, m, l = fn(ch.gc, bf16_tensor(ch.qbits), torch.from_numpy(ch.k_new).cuda(), torch.from_numpy(ch.v_new).cuda(),
                 torch.from_numpy(pt_gpu).cuda(), ch.pos0, SM)
    torch.cuda.synchronize()
    after = (ch.gc.k_nib, ch.gc.k_scale, ch.gc.v_nib, ch.gc.v_scale)
    for name, a, b in zip(("k_nib", "k_scale", "v_nib", "v_scale"), before, after):
        assert torch.equal(a, b), f"{name} changed"
    # every row sees the 128 cached tokens only
    o = o.cpu().numpy()
    qv = bf16_values(ch.qbits)
    for i in range(0, ch.T, 9):
        if fp8:
            # the 8-bit model of a query at position 127: the same 128 keys, the same groups
            ro, _, _ = ofp8.prefill(ch.oc, qv[i:i + 1], ch.pt[:2], ch.pos0 - 1, SM)
            assert_attention_close(o[i], ro[0], f"8-bit prefill row {i}")
            continue
        for g in range(4):
            K, V = oatt.gather_values(ch.oc, ch.pt, ch.pos0, g)
            ro, _, _ = oatt.decode_head_from_values(qv[i, 4 * g:4 * g + 4], K, V, SM)
            assert_attention_close(o[i, 4 * g:4 * g + 4], ro[0], f"prefill row {i} kv head {g}")
