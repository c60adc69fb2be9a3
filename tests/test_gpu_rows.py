"""paged_attn_decode_rows_f4 (R query rows per sequence, as a speculative
verification round takes them) on the GPU vs the oracle (max |delta| <= 2e-3 x
output RMS)."""
import numpy as np
import pytest
import torch

import long_context_attention_kv_amd as f4
import synth
from oracle import attention as oatt
from gpu_cases import PagedSet, assert_attention_close, assert_states_close, bf16_tensor, bf16_values

pytestmark = pytest.mark.gpu
SM = 1.0 / 16.0


def _q(B, R, Hq, seed):
    g = synth.rng(900 + seed, 1)
    bits = synth.f32_to_bf16_bits(synth.normal_f32(g, (B, R, Hq, 256)))
    return bits, bf16_values(bits)


def _run(ps, R, Hq, seed, W=1, wt=0):
    bits, qv = _q(len(ps.lengths), R, Hq, seed)
    out, m, l = f4.paged_attn_decode_rows_f4(ps.gc, bf16_tensor(bits), ps.gpu_page_table(), ps.gpu_lengths(),
                                             max(ps.lengths), SM, num_windows=W, window_tokens=wt)
    torch.cuda.synchronize()
    ro, rm, rl = oatt.decode_rows(ps.oc, qv, ps.pt, ps.lengths, SM, window_tokens=wt, num_windows=W)
    return (out.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()), (ro, rm, rl), bits


@pytest.mark.parametrize("R", [2, 3, 5, 8])
def test_rows_group_of_four(R):
    # 4 query heads per KV head: 2 rows run on the decode kernel in one pass over the pages, 3 in two;
    # 5 and more rows of a whole-context call go through the prefill kernel
    ps = PagedSet([700, 130, 64 * 20 + 5], Hkv=4, seed=900 + R)
    (o, m, l), (ro, rm, rl), _ = _run(ps, R, 16, R)
    assert_attention_close(o, ro, f"R={R}")
    assert_states_close(m, l, rm, rl, f"R={R}")


@pytest.mark.parametrize("G,Hkv,R", [(1, 2, 8), (2, 2, 3), (8, 2, 2)])
def test_rows_other_groups(G, Hkv, R):
    ps = PagedSet([300, 1024], Hkv=Hkv, seed=910 + G, v_per_token=(G == 2))
    (o, m, l), (ro, rm, rl), _ = _run(ps, R, G * Hkv, 10 + G)
    assert_attention_close(o, ro, f"G={G} R={R}")
    assert_states_close(m, l, rm, rl, f"G={G} R={R}")


def test_rows_short_contexts_and_windows():
    # contexts shorter than R: the leading rows see no token and are the merge identity
    ps = PagedSet([3, 1, 1500], Hkv=4, seed=920)
    (o, m, l), (ro, rm, rl), _ = _run(ps, 4, 16, 20, W=3, wt=640)
    assert np.all(np.isneginf(m[:, 1, :3])) and np.all(l[:, 1, :3] == 0) and not o[:, 1, :3].any()
    assert_attention_close(o, ro, "short contexts, windows")
    assert_states_close(m, l, rm, rl, "short contexts, windows")


def test_one_row_is_plain_decode_and_last_row_matches_decode():
    ps = PagedSet([2000, 77], Hkv=4, seed=930)
    bits, _ = _q(2, 5, 16, 30)
    pt, lens = ps.gpu_page_table(), ps.gpu_lengths()
    one = f4.paged_attn_decode_rows_f4(ps.gc, bf16_tensor(bits[:, 4:5].copy()), pt, lens, 2000, SM)[0]
    dec = f4.paged_attn_decode_f4(ps.gc, bf16_tensor(bits[:, 4].copy()), pt, lens, 2000, SM)[0]
    # two and three rows run on the decode kernel too (its products, to within fp32 summation order);
    # five rows on the prefill kernel (its own products, within the attention tolerance)
    two = f4.paged_attn_decode_rows_f4(ps.gc, bf16_tensor(bits[:, 3:5].copy()), pt, lens, 2000, SM)[0]
    three = f4.paged_attn_decode_rows_f4(ps.gc, bf16_tensor(bits[:, 2:5].copy()), pt, lens, 2000, SM)[0]
    five = f4.paged_attn_decode_rows_f4(ps.gc, bf16_tensor(bits), pt, lens, 2000, SM)[0]
    torch.cuda.synchronize()
    assert torch.equal(one[:, :, 0], dec)
    tol = 1e-5 * float(dec.abs().max())
    assert torch.allclose(two[:, :, 1], dec, rtol=0, atol=tol)
    assert torch.allclose(three[:, :, 2], dec, rtol=0, atol=tol)
    assert_attention_close(five[:, :, 4].cpu().numpy(), dec.cpu().numpy(), "last of five rows vs decode")


@pytest.mark.parametrize("v_per_token", [False, True])
def test_rows_through_the_prefill_kernel_short_contexts(v_per_token):
    """Rows of whole-context calls with R >= 5 (group of 4) run on the prefill
    kernel: contexts shorter than R leave the leading rows empty (the merge
    identity), an empty context all of them."""
    print(f"rows via prefill, short contexts, v_per_token={v_per_token}", flush=True)
    ps = PagedSet([3, 1, 1500, 64, 0], Hkv=4, seed=940, v_per_token=v_per_token)
    (o, m, l), (ro, rm, rl), _ = _run(ps, 8, 16, 40)
    assert np.all(np.isneginf(m[0, 0, :5])) and np.all(l[0, 0, :5] == 0) and not o[0, 0, :5].any()
    assert np.all(np.isneginf(m[0, 4])) and np.all(l[0, 4] == 0) and not o[0, 4].any()
    assert_attention_close(o, ro, "rows via prefill, short contexts")
    assert_states_close(m, l, rm, rl, "rows via prefill, short contexts")


def test_rows_through_the_prefill_kernel_agree_with_the_decode_kernel():
    """The same 6 rows through the prefill kernel (whole context) and through the
    decode kernel (one window that covers the context)."""
    print("rows via prefill vs decode kernel", flush=True)
    ps = PagedSet([2000, 300, 4097], Hkv=4, seed=950)
    bits, qv = _q(3, 6, 16, 50)
    pt, lens = ps.gpu_page_table(), ps.gpu_lengths()
    a = f4.paged_attn_decode_rows_f4(ps.gc, bf16_tensor(bits), pt, lens, 4097, SM)
    b = f4.paged_attn_decode_rows_f4(ps.gc, bf16_tensor(bits), pt, lens, 4097, SM, num_windows=1,
                                     window_tokens=64 * 65)
    torch.cuda.synchronize()
    a = [x.cpu().numpy() for x in a]
    b = [x.cpu().numpy() for x in b]
    assert_attention_close(a[0], b[0], "prefill kernel vs decode kernel")
    assert_states_close(a[1], a[2], b[1], b[2], "prefill kernel vs decode kernel")
    ro, rm, rl = oatt.decode_rows(ps.oc, qv, ps.pt, ps.lengths, SM)
    assert_attention_close(a[0], ro, "prefill kernel vs oracle")


def test_rows_through_the_prefill_kernel_drop_out_of_range_pages():
    """Out-of-range page ids on the prefill kernel's verification route (R = 5):
    those pages' tokens are dropped; each row's expected result is the oracle's
    attention over the remaining tokens up to its position."""
    print("rows via prefill, out-of-range page ids", flush=True)
    R = 5
    ps = PagedSet([1300, 200], Hkv=4, seed=960)
    pt = ps.pt.copy()
    dropped = {0: [0, 9], 1: [2]}
    pt[0, 0] = ps.num_pages + 3
    pt[0, 9] = -1
    pt[1, 2] = -5
    bits, qv = _q(2, R, 16, 60)
    out, m, l = f4.paged_attn_decode_rows_f4(ps.gc, bf16_tensor(bits), torch.from_numpy(pt).cuda(),
                                             ps.gpu_lengths(), 1300, SM)
    torch.cuda.synchronize()
    out, m, l = out.cpu().numpy()[0], m.cpu().numpy()[0], l.cpu().numpy()[0]
    for b, n in enumerate(ps.lengths):
        keep = np.ones(n, bool)
        for lp in dropped[b]:
            keep[lp * 64:(lp + 1) * 64] = False
        for g in range(4):
            K, V = oatt.gather_values(ps.oc, ps.pt[b], n, g)
            for r in range(R):
                sel = keep & (np.arange(n) <= n - R + r)
                ro, rm, rl = oatt.decode_head_from_values(qv[b, r, 4 * g:4 * g + 4], K[sel], V[sel], SM)
                hs = slice(4 * g, 4 * g + 4)
                assert_attention_close(out[b, r, hs], ro[0], f"rows b={b} r={r} kv head {g}")
                assert_states_close(m[b, r, hs], l[b, r, hs], rm[0], rl[0], f"rows b={b} r={r} g={g}")
