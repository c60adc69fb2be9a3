"""F4 paged attention with YaRN rope for MI355X (gfx950).

A thin Python binding over the C ABI of ``libf4kv.so`` (declared in
``include/f4kv.h``).  Every step of the computation runs in the library's HIP
kernels; this module only turns torch tensors into pointers, sizes and the
current stream, allocates outputs and workspaces with torch, and raises
``F4KVError`` with the library's message when a call is refused.  If the
library is not built the calls raise; there is no other code path.
"""
from ._binding import (  # noqa: F401
    CHECK_CONTEXT,
    CHECK_PAGE,
    CHECK_ROWS,
    CHECK_SLOT,
    KERNEL_DECODE,
    KERNEL_PREFILL,
    KERNEL_PREFILL_FP8,
    F4KVError,
    F4Cache,
    KernelTimer,
    YarnParams,
    abi_version,
    cache_bytes,
    decode_rows_workspace_size,
    decode_workspace_size,
    device_check_word,
    device_checks,
    gather_kv_cache_f4,
    kv_cache_write_f4,
    library_path,
    load_library,
    lse_merge,
    paged_attn_decode_f4,
    paged_attn_decode_f4_noalloc,
    paged_attn_decode_step_f4,
    paged_attn_decode_rows_f4,
    paged_attn_prefill_f4,
    paged_attn_prefill_f4_fp8,
    prefill_workspace_size,
    yarn_rope_apply,
    yarn_rope_table,
)

EXPORTED_SYMBOLS = (
    "f4kv_abi_version",
    "f4kv_last_error",
    "f4kv_cache_bytes",
    "yarn_rope_table",
    "yarn_rope_apply",
    "kv_cache_write_f4",
    "paged_attn_decode_f4_workspace_size",
    "paged_attn_decode_f4",
    "paged_attn_decode_f4_noalloc",
    "paged_attn_decode_step_f4",
    "paged_attn_decode_rows_f4_workspace_size",
    "paged_attn_decode_rows_f4",
    "lse_merge",
    "paged_attn_prefill_f4_workspace_size",
    "paged_attn_prefill_f4",
    "paged_attn_prefill_f4_fp8",
    "gather_kv_cache_f4",
    "f4kv_device_checks",
    "f4kv_device_check_word",
    "f4kv_timing_start",
    "f4kv_timing_stop",
)
