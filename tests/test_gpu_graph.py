"""The decode step captured in a HIP graph, as separate calls and as the
one-call step: every replay equals the eager result (of the separate calls).

The library's launches go on the caller's stream and use no memset nodes, so a
captured step (YaRN rows, query and key rotation, F4 write, decode with its
query preparation and fold) replays bit for bit.  Each replay is checked
against the eager outputs, with eager work and synchronisation in between.
"""
import numpy as np
import pytest
import torch

import long_context_attention_kv_amd as f4
from gpu_cases import PagedSet, bf16_tensor, random_q

pytestmark = pytest.mark.gpu
SM = 1.0 / 16.0


@pytest.mark.parametrize("one_call", [False, True])
def test_decode_step_graph_replays_match_eager(one_call):
    ps = PagedSet([5000, 777, 3000], Hkv=4, seed=21, extra_pages=8)
    bits, _ = random_q(3, 16, 256, 21)
    q_raw = bf16_tensor(bits)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    k_new = torch.randn((3, 4, 256), generator=g, device="cuda")
    v_new = torch.randn((3, 4, 256), generator=g, device="cuda")
    lens = ps.gpu_lengths()
    pos = (lens - 1).to(torch.int32)
    pt = ps.gpu_page_table()
    slots = (pt[torch.arange(3, device="cuda"), (pos // 64).long()].to(torch.int64) * 64 + pos % 64).to(torch.int32)
    yp = f4.YarnParams(factor=4.0)
    ws = torch.empty(max(16, f4.decode_workspace_size(3, 16, 4, 256, 5000)), dtype=torch.uint8, device="cuda")
    out = torch.empty((1, 3, 16, 256), device="cuda")
    om = torch.empty((1, 3, 16), device="cuda")
    ol = torch.empty((1, 3, 16), device="cuda")

    def step(one=False):
        c, s = f4.yarn_rope_table(yp, pos)
        if one:  # the one-call step: the same results, bit for bit
            f4.paged_attn_decode_step_f4(ps.gc, c, s, q_raw, k_new, v_new, slots, pt, lens, 5000, SM, out=out,
                                         out_m=om, out_l=ol, workspace=ws)
            return
        q = f4.yarn_rope_apply(c, s, q_raw)
        k = f4.yarn_rope_apply(c, s, k_new)
        f4.kv_cache_write_f4(ps.gc, k, v_new, slots)
        f4.paged_attn_decode_f4(ps.gc, q, pt, lens, 5000, SM, out=out, out_m=om, out_l=ol, workspace=ws)

    print(f"graph replays, {'one-call step' if one_call else 'separate calls'}", flush=True)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, om, ol)]
    assert torch.isfinite(ref[0]).all()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step(one_call)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            step(one_call)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (out, om, ol):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "m", "l"), (out, om, ol), ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
        # eager work between replays, on other buffers
        other = f4.paged_attn_decode_f4(ps.gc, q_raw, pt, lens, 5000, SM)[0]
        torch.cuda.synchronize()
        assert np.isfinite(other.cpu().numpy()).all()
