"""The device-side checks of values the host cannot see: each entry point, with
the checks on, raises the flag of the bad value it was given (and still skips
the value as without checks); good inputs raise nothing; with the checks off
nothing is raised."""
import pytest
import torch

import long_context_attention_kv_amd as f4
from gpu_cases import PagedSet, bf16_tensor, random_q
from test_gpu_prefill import Chunk, PAGE, SM

pytestmark = pytest.mark.gpu


@pytest.fixture()
def checks():
    f4.device_check_word()  # clear
    f4.device_checks(True)
    yield
    f4.device_checks(False)
    f4.device_check_word()


def _decode(ps, pt, lengths, max_ctx):
    bits, _ = random_q(len(lengths), 16, 256, seed=5)
    f4.paged_attn_decode_f4(ps.gc, bf16_tensor(bits), torch.from_numpy(pt).cuda(),
                            torch.tensor(lengths, dtype=torch.int32, device="cuda"), max_ctx, SM)


def test_good_inputs_raise_nothing(checks):
    print("device checks: valid decode, prefill, write, gather", flush=True)
    ps = PagedSet([700, 300], seed=41)
    _decode(ps, ps.pt, ps.lengths, 700)
    ch = Chunk(100, 40, seed=41)
    ch.run_gpu()
    total = sum(ps.lengths)
    cu = torch.tensor([0, 700, 1000], dtype=torch.int32, device="cuda")
    f4.gather_kv_cache_f4(ps.gc, ps.gpu_page_table(), cu, total)
    assert f4.device_check_word() == 0


def test_bad_values_raise_their_flags(checks):
    print("device checks: a bad page id, context length, slot id and row offset", flush=True)
    ps = PagedSet([700, 300], seed=42)
    pt = ps.pt.copy()
    pt[0, 3] = ps.num_pages + 9               # a live page of sequence 0
    _decode(ps, pt, ps.lengths, 700)
    assert f4.device_check_word() == f4.CHECK_PAGE
    _decode(ps, ps.pt, [700, 5000], 700)      # a context length past max_context_len
    # (clamped to 700, the row of the 300-token sequence has unset entries among its
    # now live pages, so the page flag may come too)
    assert f4.device_check_word() & f4.CHECK_CONTEXT
    pt2 = ps.pt.copy()
    pt2[1, 5] = -3                            # page 5 of a 300-token sequence is not live: no flag
    _decode(ps, pt2, ps.lengths, 700)
    assert f4.device_check_word() == 0
    # the writer: one slot past the pool, one -1 (skipped, fine)
    k = torch.zeros((2, 4, 256), device="cuda")
    slots = torch.tensor([ps.num_pages * PAGE + 1, -1], dtype=torch.int32, device="cuda")
    f4.kv_cache_write_f4(ps.gc, k, k, slots)
    assert f4.device_check_word() == f4.CHECK_SLOT
    # the gather: decreasing offsets
    cu = torch.tensor([0, 700, 600], dtype=torch.int32, device="cuda")
    f4.gather_kv_cache_f4(ps.gc, ps.gpu_page_table(), cu, 1000)
    assert f4.device_check_word() & f4.CHECK_ROWS
    # the prefill: a page of the chunk out of range
    ch = Chunk(100, 40, seed=42)
    ch.pt = ch.pt.copy()
    ch.pt[2] = ch.P + 4
    ch.run_gpu()
    assert f4.device_check_word() == f4.CHECK_PAGE


def test_checks_off_raise_nothing():
    print("device checks off: bad inputs raise nothing", flush=True)
    f4.device_checks(False)
    f4.device_check_word()
    ps = PagedSet([700], seed=43)
    pt = ps.pt.copy()
    pt[0, 3] = -1
    _decode(ps, pt, ps.lengths, 700)
    assert f4.device_check_word() == 0
