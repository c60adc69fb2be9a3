"""The C ABI library loads, exports every declared symbol, and refuses bad arguments on the host.

These run without a GPU: every call below fails validation before any HIP work.
"""
import ctypes as C
import os
import re

import pytest

import long_context_attention_kv_amd as f4
from long_context_attention_kv_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "f4kv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(f4.library_path()):
        import long_context_attention_kv_amd.build as bld
        bld.build()
    return f4.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 21, names
    assert set(names) == set(f4.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(lib):
    src = open(HEADER).read()
    v = int(re.search(r"#define F4KV_ABI_VERSION (\d+)", src).group(1))
    assert lib.f4kv_abi_version() == v


def test_cache_bytes(lib):
    total, parts = f4.cache_bytes(16384, 4, 256)
    # per token and KV head: 128 bytes of nibbles + 8 fp16 scales, for K and for V
    assert parts == (16384 * 4 * 64 * 128, 16384 * 4 * 64 * 16, 16384 * 4 * 64 * 128, 16384 * 4 * 64 * 16)
    assert total == 16384 * 64 * 4 * 2 * 144
    assert lib.f4kv_cache_bytes(1, 1, 48, 0, None, None, None, None) == 0
    assert lib.f4kv_cache_bytes(1, 1, 256, 2, None, None, None, None) == 0
    # one V scale per token and head: 130 bytes of V per token and head
    total, parts = f4.cache_bytes(16384, 4, 256, v_scale_per_token=True)
    assert parts == (16384 * 4 * 64 * 128, 16384 * 4 * 64 * 16, 16384 * 4 * 64 * 128, 16384 * 4 * 64 * 2)
    assert total == 16384 * 64 * 4 * (144 + 130)


def _cache(ptr=16, pages=8, heads=4, dim=256, page=64, vtok=0):
    return B._CacheC(ptr, ptr, ptr, ptr, pages, heads, dim, page, vtok)


def _yarn(**kw):
    d = dict(theta=1e7, rotary_dim=256, factor=4.0, orig_ctx=262144, beta_fast=32.0, beta_slow=1.0, mscale=0.0)
    d.update(kw)
    return B._YarnParamsC(**d)


def _err(lib):
    return lib.f4kv_last_error().decode()


@pytest.mark.parametrize("kw,needle", [
    (dict(factor=0.5), "factor"),
    (dict(factor=64.5), "factor"),
    (dict(rotary_dim=255), "rotary_dim"),
    (dict(theta=1.0), "theta"),
    (dict(beta_fast=1.0, beta_slow=32.0), "beta"),
    (dict(orig_ctx=0), "orig_ctx"),
])
def test_yarn_params_refused(lib, kw, needle):
    p = _yarn(**kw)
    r = lib.yarn_rope_table(C.byref(p), 16, 4, 16, 16, None)
    assert r == 1 and needle in _err(lib)


def test_yarn_factor_range_edges(lib):
    # factor 64 is the largest accepted (ignis --model-rope-scaling: F in (1, 64]); n == 0 is a no-op
    p = _yarn(factor=64.0)
    assert lib.yarn_rope_table(C.byref(p), None, 0, None, None, None) == 0
    p = _yarn(factor=1.0)
    assert lib.yarn_rope_table(C.byref(p), None, 0, None, None, None) == 0
    p = _yarn(factor=4.0)
    assert lib.yarn_rope_table(C.byref(p), None, 5, None, None, None) == 1


@pytest.mark.parametrize("field,val,needle", [
    ("page_size", 32, "page_size"),
    ("head_dim", 48, "head_dim"),
    ("num_pages", 0, "num_pages"),
    ("k_nib", 0, "NULL"),
    ("v_scale", 8, "aligned"),
    ("v_scale_per_token", 2, "v_scale_per_token"),
])
def test_cache_descriptor_refused(lib, field, val, needle):
    c = _cache()
    setattr(c, field, val)
    r = lib.kv_cache_write_f4(C.byref(c), 16, 16, 16, 1, None)
    assert r == 1 and needle in _err(lib)


def test_writer_argument_checks(lib):
    c = _cache()
    assert lib.kv_cache_write_f4(C.byref(c), 16, 16, 16, 0, None) == 0          # empty: nothing to do
    assert lib.kv_cache_write_f4(C.byref(c), None, 16, 16, 3, None) == 1
    assert lib.kv_cache_write_f4(C.byref(c), 20, 16, 16, 3, None) == 1           # k misaligned
    assert lib.kv_cache_write_f4(C.byref(c), 16, 16, 16, -1, None) == 1
    assert lib.kv_cache_write_f4(None, 16, 16, 16, 1, None) == 1


def _decode(lib, c, B_=1, Hq=16, max_pages=64, max_ctx=4096, W=1, wt=0, ws=None, ws_bytes=0, q=16, out=16):
    return lib.paged_attn_decode_f4(C.byref(c), q, 16, 16, B_, Hq, max_pages, max_ctx, W, wt, 0.0625, out, None,
                                    None, ws, ws_bytes, None)


def test_decode_argument_checks(lib):
    c = _cache()
    assert _decode(lib, c, Hq=6) == 1 and "multiple" in _err(lib)
    assert _decode(lib, c, max_ctx=64 * 64 + 1) == 1 and "max_pages" in _err(lib)
    assert _decode(lib, c, W=4, wt=0) == 1 and "window" in _err(lib)
    assert _decode(lib, c, W=2, wt=100) == 1 and "64" in _err(lib)
    assert _decode(lib, c, Hq=12) == 2 and "1, 2, 4 or 8" in _err(lib)
    c128 = _cache(dim=128)
    assert _decode(lib, c128) == 2 and "head_dim" in _err(lib)
    assert _decode(lib, c, q=8) == 1 and "aligned" in _err(lib)
    assert _decode(lib, c, B_=0) == 0
    need = lib.paged_attn_decode_f4_workspace_size(1, 16, 4, 256, 1 << 20, 16, 65536)
    assert need > 0
    assert _decode(lib, c, max_pages=16384, max_ctx=1 << 20, W=16, wt=65536, ws=16, ws_bytes=need - 1) == 3
    assert "workspace" in _err(lib)
    assert _decode(lib, c, max_pages=16384, max_ctx=1 << 20, W=16, wt=65536, ws=None, ws_bytes=need) == 3


def _step(lib, c, B_=1, rd=256, tables=16, kv=16, slots=16, **kw):
    return lib.paged_attn_decode_step_f4(C.byref(c), tables, tables, rd, 16, kv, kv, slots, 16, 16, B_, 16, 64, 4096,
                                         1, 0, 0.0625, 16, None, None, kw.get("ws"), kw.get("ws_bytes", 0), None)


def test_decode_step_argument_checks(lib):
    """The one-call decode step refuses bad rotation and new-token arguments on
    the host, besides the decode's own checks; nothing is launched."""
    c = _cache()
    assert _step(lib, c, rd=0) == 1 and "rotary_dim" in _err(lib)
    assert _step(lib, c, rd=255) == 1 and "rotary_dim" in _err(lib)
    assert _step(lib, c, rd=258) == 1 and "rotary_dim" in _err(lib)
    assert _step(lib, c, tables=None) == 1 and "NULL" in _err(lib)
    assert _step(lib, c, slots=None) == 1 and "NULL" in _err(lib)
    assert _step(lib, c, kv=8) == 1 and "aligned" in _err(lib)
    assert _step(lib, c, slots=18) == 1 and "aligned" in _err(lib)
    assert _step(lib, _cache(dim=128), rd=128) == 2 and "head_dim" in _err(lib)
    assert _step(lib, c, B_=0, tables=None, kv=None, slots=None) == 0


def test_decode_noalloc_refuses_beyond_its_scratch(lib):
    """The allocation-free decode takes no workspace: the same argument checks,
    and a call whose workspace would exceed the fixed 8 MiB scratch is refused
    on the host (no launch, no allocation)."""
    c = _cache()

    def call(B_=1, Hq=16, max_pages=64, max_ctx=4096, W=1, wt=0, q=16):
        return lib.paged_attn_decode_f4_noalloc(C.byref(c), q, 16, 16, B_, Hq, max_pages, max_ctx, W, wt, 0.0625, 16,
                                                None, None, None)

    assert call(Hq=6) == 1 and "multiple" in _err(lib)
    assert call(W=2, wt=100) == 1 and "64" in _err(lib)
    assert call(B_=0) == 0
    need = lib.paged_attn_decode_f4_workspace_size(1, 16, 4, 256, 1 << 20, 16384, 64)
    assert need > 8 << 20
    assert call(max_pages=16384, max_ctx=1 << 20, W=16384, wt=64) == 2 and "scratch" in _err(lib)


def test_decode_rows_argument_checks(lib):
    c = _cache()
    d = lib.paged_attn_decode_rows_f4
    args = lambda R: (C.byref(c), 16, 16, 16, 1, R, 16, 64, 4096, 1, 0, 0.0625, 16, None, None, None, 0, None)
    assert d(*args(0)) == 1 and "rows" in _err(lib)
    assert d(*args(9)) == 1 and "rows" in _err(lib)
    assert d(*args(2)) == 3 and "workspace" in _err(lib)
    # more rows need more workspace; R == 1 is plain decode's size
    one = lib.paged_attn_decode_rows_f4_workspace_size(3, 1, 16, 4, 256, 1 << 18, 1, 0)
    assert one == lib.paged_attn_decode_f4_workspace_size(3, 16, 4, 256, 1 << 18, 1, 0)
    assert lib.paged_attn_decode_rows_f4_workspace_size(3, 8, 16, 4, 256, 1 << 18, 1, 0) > one
    assert lib.paged_attn_decode_rows_f4_workspace_size(3, 9, 16, 4, 256, 1 << 18, 1, 0) == 0


def test_gather_argument_checks(lib):
    c = _cache()
    g = lib.gather_kv_cache_f4
    assert g(C.byref(c), 16, 16, 0, 4, 100, 16, 16, 1, None) == 0                      # B == 0: nothing to do
    assert g(C.byref(c), 16, 16, 2, 4, 0, 16, 16, 1, None) == 0                        # no rows
    assert g(C.byref(c), 16, 16, 2, 4, 100, 16, 16, 5, None) == 1 and "out_dtype" in _err(lib)
    assert g(C.byref(c), None, 16, 2, 4, 100, 16, 16, 1, None) == 1 and "NULL" in _err(lib)
    assert g(C.byref(c), 16, 16, 2, 4, 100, 24, 16, 1, None) == 1 and "aligned" in _err(lib)
    assert g(C.byref(c), 16, 16, 70000, 4, 100, 16, 16, 1, None) == 1
    assert g(C.byref(c), 16, 16, 2, 0, 100, 16, 16, 1, None) == 1 and "max_pages" in _err(lib)
    wide = _cache(heads=128)                                                             # grid of max_pages * H
    assert g(C.byref(wide), 16, 16, 2, 1 << 24, 100, 16, 16, 1, None) == 1 and "num_kv_heads" in _err(lib)
    c64 = _cache(dim=64)
    assert g(C.byref(c64), 16, 16, 2, 4, 100, 16, 16, 1, None) == 2 and "head_dim" in _err(lib)


def test_merge_and_rope_apply_checks(lib):
    assert lib.lse_merge(16, 16, 16, 0, 4, 256, 16, None, None, None) == 1
    assert lib.lse_merge(16, 16, 16, 2, 4, 250, 16, None, None, None) == 1
    assert lib.lse_merge(16, 16, 16, 2, 0, 256, 16, None, None, None) == 0
    assert lib.yarn_rope_apply(16, 16, 16, 2, 16, 0, 1, 1, 256, 256, None) == 1   # bad dtype
    assert lib.yarn_rope_apply(16, 16, 16, 0, 16, 0, 1, 1, 256, 300, None) == 1   # rotary_dim > D
    assert lib.yarn_rope_apply(16, 16, 16, 0, 16, 1, 1, 1, 256, 256, None) == 1   # in place, dtypes differ


@pytest.mark.parametrize("name", ["paged_attn_prefill_f4", "paged_attn_prefill_f4_fp8"])
def test_prefill_argument_checks(lib, name):
    c = _cache()
    f = lambda **kw: getattr(lib, name)(
        C.byref(c), 16, kw.get("k", 16), kw.get("v", 16), 16, kw.get("mp", 64), kw.get("T", 64), kw.get("Hq", 16),
        kw.get("pos0", 0), kw.get("sm", 0.0625), 16, None, None, None, 0, None)
    assert f(pos0=64 * 64) == 1 and "max_pages" in _err(lib) and name + ":" in _err(lib)
    assert f(k=None) == 1 and "together" in _err(lib)
    assert f(sm=float("nan")) == 1 and "sm_scale" in _err(lib)
    assert f(Hq=8) == 2
    assert f(T=0) == 0


def test_timing_argument_checks(lib):
    assert lib.f4kv_timing_start(7, 16) == 1 and "unknown kernel" in _err(lib)
    assert lib.f4kv_timing_start(3, 16) == 1 and "unknown kernel" in _err(lib)
    assert lib.f4kv_timing_start(0, 0) == 1 and "max_launches" in _err(lib)
    assert lib.f4kv_timing_start(1, (1 << 20) + 1) == 1
    ms, n = C.c_double(-1.0), C.c_int64(-1)
    assert lib.f4kv_timing_stop(-1, C.byref(ms), C.byref(n)) == 1 and "unknown kernel" in _err(lib)
    # stopping a timer that never started reports no launches and touches no device
    assert lib.f4kv_timing_stop(0, C.byref(ms), C.byref(n)) == 0
    assert ms.value == 0.0 and n.value == 0


def test_device_checks_switch(lib):
    """The switch takes 0 or 1 and launches nothing by itself; the word query
    refuses a null pointer (reading the word needs a GPU: the GPU tests)."""
    assert lib.f4kv_device_checks(2) == 1 and "0 or 1" in _err(lib)
    assert lib.f4kv_device_checks(1) == 0
    assert lib.f4kv_device_checks(0) == 0
    assert lib.f4kv_device_check_word(None) == 1 and "NULL" in _err(lib)
