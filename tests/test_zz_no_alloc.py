"""paged_attn_decode_f4_noalloc (the decode on the library's fixed device-side
scratch, for callers that cannot allocate) against paged_attn_decode_f4 with a
workspace: the same kernels and plan, so the outputs must be equal bit for bit;
and against the oracle at the attention bar.  Two calls in a row, the second
with a smaller input, share the scratch."""
import numpy as np
import pytest
import torch

import long_context_attention_kv_amd as f4
from gpu_cases import PagedSet, assert_attention_close, bf16_tensor, oracle_decode, random_q

pytestmark = pytest.mark.gpu
SM = 1.0 / 16.0


def _both(ps, bits, max_ctx, W=1, wt=0):
    q = bf16_tensor(bits)
    ref = f4.paged_attn_decode_f4(ps.gc, q, ps.gpu_page_table(), ps.gpu_lengths(), max_ctx, SM, num_windows=W,
                                  window_tokens=wt)
    B, Hq = bits.shape[0], bits.shape[1]
    out = torch.full((W, B, Hq, 256), float("nan"), device="cuda")
    om = torch.full((W, B, Hq), float("nan"), device="cuda")
    ol = torch.full((W, B, Hq), float("nan"), device="cuda")
    got = f4.paged_attn_decode_f4_noalloc(ps.gc, q, ps.gpu_page_table(), ps.gpu_lengths(), max_ctx, SM,
                                          num_windows=W, window_tokens=wt, out=out, out_m=om, out_l=ol)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ref], [t.cpu().numpy() for t in got]


def test_noalloc_equals_workspace_decode_two_calls():
    print("noalloc decode: 3 sequences (5,000 / 3,000 / 2,373 tokens), then 1 sequence of 700", flush=True)
    ps = PagedSet([5000, 3000, 64 * 37 + 5], Hkv=4, seed=70, outliers=True)
    bits, qv = random_q(3, 16, 256, seed=70)
    (ro, rm, rl), (go, gm, gl) = _both(ps, bits, 5000)
    assert np.array_equal(go, ro) and np.array_equal(gm, rm) and np.array_equal(gl, rl)
    oo, _, _ = oracle_decode(ps, qv, SM)
    assert_attention_close(go, oo, "noalloc decode, first call")

    ps2 = PagedSet([700], Hkv=4, seed=71)
    bits2, qv2 = random_q(1, 16, 256, seed=71)
    (ro, rm, rl), (go, gm, gl) = _both(ps2, bits2, 700)
    assert np.array_equal(go, ro) and np.array_equal(gm, rm) and np.array_equal(gl, rl)
    oo, _, _ = oracle_decode(ps2, qv2, SM)
    assert_attention_close(go, oo, "noalloc decode, second (smaller) call")


def test_noalloc_windows_and_refusal():
    print("noalloc decode: 4 windows of 1,024 tokens; an oversized call is refused", flush=True)
    ps = PagedSet([3500, 900], Hkv=4, seed=72)
    bits, qv = random_q(2, 16, 256, seed=72)
    (ro, rm, rl), (go, gm, gl) = _both(ps, bits, 3500, W=4, wt=1024)
    assert np.array_equal(go, ro) and np.array_equal(gm, rm) and np.array_equal(gl, rl)
    oo, _, _ = oracle_decode(ps, qv, SM, num_windows=4, window_tokens=1024)
    assert_attention_close(go, oo, "noalloc decode, windows")
    # a workspace beyond the fixed scratch: 16,384 windows of one sequence
    with pytest.raises(f4.F4KVError) as e:
        f4.paged_attn_decode_f4_noalloc(ps.gc, bf16_tensor(bits[:1]), ps.gpu_page_table()[:1],
                                        ps.gpu_lengths()[:1], 3500, SM, num_windows=16384, window_tokens=64)
    assert e.value.status == 2 and "scratch" in str(e.value)
