"""gather_kv_cache_f4 on the GPU vs the oracle: bit for bit (fp32 rows are the
exact values (nibble - 8) * scale, bf16 rows those values rounded to nearest-even)."""
import numpy as np
import pytest
import torch

import long_context_attention_kv_amd as f4
import synth
from oracle import f4 as of4
from gpu_cases import PagedSet

pytestmark = pytest.mark.gpu


def _cu(lengths):
    return torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device="cuda")


def _bits(x: torch.Tensor) -> np.ndarray:
    return x.view(torch.int16).cpu().numpy() if x.dtype == torch.bfloat16 else x.view(torch.int32).cpu().numpy()


def _expect(vals: np.ndarray, dtype) -> np.ndarray:
    if dtype == torch.bfloat16:
        return torch.from_numpy(of4.bf16_round(vals).astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    return vals.astype(np.float32).view(np.int32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("vt", [False, True])
@pytest.mark.parametrize("lengths", [[1], [64], [65, 0, 700], [64 * 37 + 5, 3, 130]])
def test_gather_bit_exact(lengths, vt, dtype):
    ps = PagedSet(lengths, Hkv=4, seed=800 + sum(lengths), outliers=True, v_per_token=vt)
    total = sum(lengths)
    k, v = f4.gather_kv_cache_f4(ps.gc, ps.gpu_page_table(), _cu(lengths), total, dtype=dtype)
    torch.cuda.synchronize()
    K, V = ps.oc.gather(ps.pt, lengths)
    assert np.array_equal(_bits(k), _expect(K, dtype))
    assert np.array_equal(_bits(v), _expect(V, dtype))


def test_gather_invalid_pages_and_rows_past_total():
    lengths = [200, 100]
    ps = PagedSet(lengths, Hkv=4, seed=810)
    pt = ps.pt.copy()
    pt[0, 1] = ps.num_pages + 7     # outside the pool: zero rows
    pt[1, 0] = -1
    total = 250                     # the second sequence's last 50 rows are not written
    k = torch.full((total, 4, 256), 3.0, dtype=torch.float32, device="cuda")
    v = torch.full((total, 4, 256), 3.0, dtype=torch.float32, device="cuda")
    f4.gather_kv_cache_f4(ps.gc, torch.from_numpy(pt).cuda(), _cu(lengths), total, dtype=torch.float32,
                          k_out=k, v_out=v)
    torch.cuda.synchronize()
    K, V = ps.oc.gather(pt, lengths)
    assert np.array_equal(k.cpu().numpy(), K[:total].astype(np.float32))
    assert np.array_equal(v.cpu().numpy(), V[:total].astype(np.float32))
    assert not k[64:128].any() and not k[200:250].any()


def test_gather_matches_the_attention_path():
    # decode over a cache equals textbook attention over the gathered fp32 rows
    lengths = [3000]
    ps = PagedSet(lengths, Hkv=4, seed=820)
    k, v = f4.gather_kv_cache_f4(ps.gc, ps.gpu_page_table(), _cu(lengths), 3000, dtype=torch.float32)
    g = synth.rng(820, 5)
    q = torch.from_numpy(synth.normal_f32(g, (1, 16, 256))).cuda().to(torch.bfloat16)
    out = f4.paged_attn_decode_f4(ps.gc, q, ps.gpu_page_table(), ps.gpu_lengths(), 3000, 1 / 16)[0][0, 0]
    K = k.double().cpu().repeat_interleave(4, dim=1).transpose(0, 1)  # [16, 3000, 256]
    V = v.double().cpu().repeat_interleave(4, dim=1).transpose(0, 1)
    s = torch.einsum("hd,htd->ht", q[0].double().cpu(), K) / 16
    ref = torch.einsum("ht,htd->hd", torch.softmax(s, dim=-1), V)
    rms = ref.pow(2).mean().sqrt()
    assert (out.double().cpu() - ref).abs().max() <= 2e-3 * rms
