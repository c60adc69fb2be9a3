"""ctypes marshalling for libf4kv.so: tensors -> pointers, sizes and the current stream."""
from __future__ import annotations

import ctypes as C
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libf4kv.so")
_lib = None

F32, BF16 = 0, 1
PAGE = 64


class F4KVError(RuntimeError):
    """A call the library refused (status != 0), with its reason."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed (status {status}): {msg}")
        self.status = status


class _YarnParamsC(C.Structure):
    _fields_ = [("theta", C.c_double), ("rotary_dim", C.c_int32), ("factor", C.c_double),
                ("orig_ctx", C.c_int32), ("beta_fast", C.c_double), ("beta_slow", C.c_double),
                ("mscale", C.c_double)]


class _CacheC(C.Structure):
    _fields_ = [("k_nib", C.c_void_p), ("k_scale", C.c_void_p), ("v_nib", C.c_void_p),
                ("v_scale", C.c_void_p), ("num_pages", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("page_size", C.c_int32), ("v_scale_per_token", C.c_int32)]


_P = C.c_void_p
_I = C.c_int32
_SIGS = {
    "f4kv_abi_version": (C.c_int, []),
    "f4kv_last_error": (C.c_char_p, []),
    "f4kv_cache_bytes": (C.c_size_t, [_I, _I, _I, _I, _P, _P, _P, _P]),
    "yarn_rope_table": (C.c_int, [C.POINTER(_YarnParamsC), _P, _I, _P, _P, _P]),
    "yarn_rope_apply": (C.c_int, [_P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _P]),
    "kv_cache_write_f4": (C.c_int, [C.POINTER(_CacheC), _P, _P, _P, _I, _P]),
    "paged_attn_decode_f4_workspace_size": (C.c_size_t, [_I, _I, _I, _I, _I, _I, _I]),
    "paged_attn_decode_f4": (C.c_int, [C.POINTER(_CacheC), _P, _P, _P, _I, _I, _I, _I, _I, _I, C.c_float,
                                       _P, _P, _P, _P, C.c_size_t, _P]),
    "paged_attn_decode_f4_noalloc": (C.c_int, [C.POINTER(_CacheC), _P, _P, _P, _I, _I, _I, _I, _I, _I, C.c_float,
                                               _P, _P, _P, _P]),
    "paged_attn_decode_step_f4": (C.c_int, [C.POINTER(_CacheC), _P, _P, _I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                            _I, _I, C.c_float, _P, _P, _P, _P, C.c_size_t, _P]),
    "paged_attn_decode_rows_f4_workspace_size": (C.c_size_t, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "paged_attn_decode_rows_f4": (C.c_int, [C.POINTER(_CacheC), _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, C.c_float,
                                            _P, _P, _P, _P, C.c_size_t, _P]),
    "lse_merge": (C.c_int, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P]),
    "paged_attn_prefill_f4_workspace_size": (C.c_size_t, [_I, _I, _I, _I, _I]),
    "paged_attn_prefill_f4": (C.c_int, [C.POINTER(_CacheC), _P, _P, _P, _P, _I, _I, _I, _I, C.c_float,
                                        _P, _P, _P, _P, C.c_size_t, _P]),
    "paged_attn_prefill_f4_fp8": (C.c_int, [C.POINTER(_CacheC), _P, _P, _P, _P, _I, _I, _I, _I, C.c_float,
                                            _P, _P, _P, _P, C.c_size_t, _P]),
    "gather_kv_cache_f4": (C.c_int, [C.POINTER(_CacheC), _P, _P, _I, _I, _I, _P, _P, _I, _P]),
    "f4kv_device_checks": (C.c_int, [_I]),
    "f4kv_device_check_word": (C.c_int, [C.POINTER(C.c_uint32)]),
    "f4kv_timing_start": (C.c_int, [_I, _I]),
    "f4kv_timing_stop": (C.c_int, [_I, C.POINTER(C.c_double), C.POINTER(C.c_int64)]),
}

KERNEL_DECODE, KERNEL_PREFILL, KERNEL_PREFILL_FP8 = 0, 1, 2
CHECK_CONTEXT, CHECK_PAGE, CHECK_SLOT, CHECK_ROWS = 1, 2, 4, 8


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libf4kv.so (built in-tree by ``build.py``); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run long_context_attention_kv_amd/build.py "
                           "(or __graft_entry__.build()) first")
    lib = C.CDLL(_LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise F4KVError(fn, status, _lib.f4kv_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _need(t, dtype, shape=None, name="tensor"):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda and t.numel() > 0:
        raise ValueError(f"{name} must live on the GPU")


def abi_version() -> int:
    return load_library().f4kv_abi_version()


def cache_bytes(num_pages: int, num_kv_heads: int, head_dim: int, v_scale_per_token: bool = False):
    lib = load_library()
    a, b, c, d = (C.c_size_t() for _ in range(4))
    total = lib.f4kv_cache_bytes(num_pages, num_kv_heads, head_dim, int(bool(v_scale_per_token)), C.byref(a),
                                 C.byref(b), C.byref(c), C.byref(d))
    return total, (a.value, b.value, c.value, d.value)


@dataclass
class YarnParams:
    theta: float = 1.0e7
    rotary_dim: int = 256
    factor: float = 1.0
    orig_ctx: int = 262144
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    mscale: float = 0.0

    def _c(self):
        return _YarnParamsC(float(self.theta), int(self.rotary_dim), float(self.factor), int(self.orig_ctx),
                            float(self.beta_fast), float(self.beta_slow), float(self.mscale))


class F4Cache:
    """One layer's paged F4 cache: four device tensors in the library's layout
    (``v_scale_per_token``: one V scale per token and head instead of per 32 values)."""

    def __init__(self, num_pages: int, num_kv_heads: int, head_dim: int = 256, device="cuda",
                 v_scale_per_token: bool = False):
        nb = head_dim // 32
        self.num_pages, self.num_kv_heads, self.head_dim = num_pages, num_kv_heads, head_dim
        self.v_scale_per_token = bool(v_scale_per_token)
        self.k_nib = torch.zeros((num_pages, num_kv_heads, nb, PAGE, 16), dtype=torch.uint8, device=device)
        self.k_scale = torch.zeros((num_pages, num_kv_heads, PAGE, nb), dtype=torch.int16, device=device)
        self.v_nib = torch.zeros((num_pages, num_kv_heads, PAGE // 8, head_dim // 4, 16), dtype=torch.uint8,
                                 device=device)
        vs_shape = (num_pages, num_kv_heads, PAGE) if self.v_scale_per_token else (num_pages, num_kv_heads, PAGE, nb)
        self.v_scale = torch.zeros(vs_shape, dtype=torch.int16, device=device)

    def _c(self):
        return _CacheC(self.k_nib.data_ptr(), self.k_scale.data_ptr(), self.v_nib.data_ptr(),
                       self.v_scale.data_ptr(), self.num_pages, self.num_kv_heads, self.head_dim, PAGE,
                       int(self.v_scale_per_token))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.k_nib, self.k_scale, self.v_nib, self.v_scale))


def yarn_rope_table(params: YarnParams, positions: torch.Tensor, cos_out=None, sin_out=None):
    lib = load_library()
    n = positions.numel()
    _need(positions, torch.int32, (n,), "positions")
    half = params.rotary_dim // 2
    if cos_out is None:
        cos_out = torch.empty((n, half), dtype=torch.float32, device=positions.device)
    if sin_out is None:
        sin_out = torch.empty((n, half), dtype=torch.float32, device=positions.device)
    _need(cos_out, torch.float32, (n, half), "cos_out")
    _need(sin_out, torch.float32, (n, half), "sin_out")
    p = params._c()
    _check("yarn_rope_table", lib.yarn_rope_table(C.byref(p), _ptr(positions), n, _ptr(cos_out), _ptr(sin_out),
                                                  _stream()))
    return cos_out, sin_out


def _dt(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("rope tensors must be float32 or bfloat16")


def yarn_rope_apply(cos_rows, sin_rows, x, y=None, rotary_dim=None):
    """Rotate x [T, H, D] in fp64 arithmetic; y defaults to a new tensor of x's dtype (y=x: in place)."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be [T, H, D]")
    T, H, D = x.shape
    rd = rotary_dim if rotary_dim is not None else 2 * cos_rows.shape[-1]
    _need(cos_rows, torch.float32, (T, rd // 2), "cos_rows")
    _need(sin_rows, torch.float32, (T, rd // 2), "sin_rows")
    if y is None:
        y = torch.empty_like(x)
    if not x.is_contiguous() or not y.is_contiguous() or tuple(y.shape) != tuple(x.shape):
        raise ValueError("x and y must be contiguous [T, H, D]")
    _check("yarn_rope_apply", lib.yarn_rope_apply(_ptr(cos_rows), _ptr(sin_rows), _ptr(x), _dt(x), _ptr(y), _dt(y),
                                                  T, H, D, rd, _stream()))
    return y


def kv_cache_write_f4(cache: F4Cache, k, v, slot_mapping):
    lib = load_library()
    T = k.shape[0]
    shape = (T, cache.num_kv_heads, cache.head_dim)
    _need(k, torch.float32, shape, "k")
    _need(v, torch.float32, shape, "v")
    _need(slot_mapping, torch.int32, (T,), "slot_mapping")
    c = cache._c()
    _check("kv_cache_write_f4", lib.kv_cache_write_f4(C.byref(c), _ptr(k), _ptr(v), _ptr(slot_mapping), T,
                                                      _stream()))


def decode_workspace_size(B, Hq, num_kv_heads, head_dim, max_context_len, num_windows=1, window_tokens=0) -> int:
    return load_library().paged_attn_decode_f4_workspace_size(B, Hq, num_kv_heads, head_dim, max_context_len,
                                                              num_windows, window_tokens)


def paged_attn_decode_f4(cache: F4Cache, q, page_table, context_lens, max_context_len: int, sm_scale: float,
                         num_windows: int = 1, window_tokens: int = 0, out=None, out_m=None, out_l=None,
                         workspace=None):
    """Decode attention; returns (out [W, B, Hq, D], m [W, B, Hq], l [W, B, Hq])."""
    lib = load_library()
    B, Hq, D = q.shape
    _need(q, torch.bfloat16, (B, Hq, D), "q")
    _need(page_table, torch.int32, None, "page_table")
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B, max_pages]")
    _need(context_lens, torch.int32, (B,), "context_lens")
    W = num_windows
    dev = q.device
    if out is None:
        out = torch.empty((W, B, Hq, D), dtype=torch.float32, device=dev)
    if out_m is None:
        out_m = torch.empty((W, B, Hq), dtype=torch.float32, device=dev)
    if out_l is None:
        out_l = torch.empty((W, B, Hq), dtype=torch.float32, device=dev)
    _need(out, torch.float32, (W, B, Hq, D), "out")
    ws_need = decode_workspace_size(B, Hq, cache.num_kv_heads, cache.head_dim, max_context_len, W, window_tokens)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = cache._c()
    _check("paged_attn_decode_f4",
           lib.paged_attn_decode_f4(C.byref(c), _ptr(q), _ptr(page_table), _ptr(context_lens), B, Hq,
                                    page_table.shape[1], int(max_context_len), W, int(window_tokens),
                                    float(sm_scale), _ptr(out), _ptr(out_m), _ptr(out_l), _ptr(workspace), ws_bytes,
                                    _stream()))
    return out, out_m, out_l


def paged_attn_decode_step_f4(cache: F4Cache, cos_rows, sin_rows, q, k_new, v_new, slots, page_table, context_lens,
                              max_context_len: int, sm_scale: float, num_windows: int = 1, window_tokens: int = 0,
                              rotary_dim=None, out=None, out_m=None, out_l=None, workspace=None):
    """One decode step: rotate q [B, Hq, D] (bf16) and k_new [B, Hkv, D] (fp32) with
    table rows [B, rotary_dim/2], write k and v_new at slots [B], then decode;
    returns (out [W, B, Hq, D], m [W, B, Hq], l [W, B, Hq])."""
    lib = load_library()
    B, Hq, D = q.shape
    _need(q, torch.bfloat16, (B, Hq, D), "q")
    kv_shape = (B, cache.num_kv_heads, cache.head_dim)
    _need(k_new, torch.float32, kv_shape, "k_new")
    _need(v_new, torch.float32, kv_shape, "v_new")
    _need(slots, torch.int32, (B,), "slots")
    rd = rotary_dim if rotary_dim is not None else 2 * cos_rows.shape[-1]
    _need(cos_rows, torch.float32, (B, rd // 2), "cos_rows")
    _need(sin_rows, torch.float32, (B, rd // 2), "sin_rows")
    _need(page_table, torch.int32, None, "page_table")
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B, max_pages]")
    _need(context_lens, torch.int32, (B,), "context_lens")
    W = num_windows
    dev = q.device
    if out is None:
        out = torch.empty((W, B, Hq, D), dtype=torch.float32, device=dev)
    if out_m is None:
        out_m = torch.empty((W, B, Hq), dtype=torch.float32, device=dev)
    if out_l is None:
        out_l = torch.empty((W, B, Hq), dtype=torch.float32, device=dev)
    _need(out, torch.float32, (W, B, Hq, D), "out")
    ws_need = decode_workspace_size(B, Hq, cache.num_kv_heads, cache.head_dim, max_context_len, W, window_tokens)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = cache._c()
    _check("paged_attn_decode_step_f4",
           lib.paged_attn_decode_step_f4(C.byref(c), _ptr(cos_rows), _ptr(sin_rows), int(rd), _ptr(q), _ptr(k_new),
                                         _ptr(v_new), _ptr(slots), _ptr(page_table), _ptr(context_lens), B, Hq,
                                         page_table.shape[1], int(max_context_len), W, int(window_tokens),
                                         float(sm_scale), _ptr(out), _ptr(out_m), _ptr(out_l), _ptr(workspace),
                                         ws_bytes, _stream()))
    return out, out_m, out_l


def paged_attn_decode_f4_noalloc(cache: F4Cache, q, page_table, context_lens, max_context_len: int,
                                 sm_scale: float, num_windows: int = 1, window_tokens: int = 0, out=None, out_m=None,
                                 out_l=None):
    """paged_attn_decode_f4 on the library's fixed device-side scratch (the C call
    allocates nothing; pass out, out_m, out_l to allocate nothing here either)."""
    lib = load_library()
    B, Hq, D = q.shape
    _need(q, torch.bfloat16, (B, Hq, D), "q")
    _need(page_table, torch.int32, None, "page_table")
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B, max_pages]")
    _need(context_lens, torch.int32, (B,), "context_lens")
    W = num_windows
    dev = q.device
    if out is None:
        out = torch.empty((W, B, Hq, D), dtype=torch.float32, device=dev)
    if out_m is None:
        out_m = torch.empty((W, B, Hq), dtype=torch.float32, device=dev)
    if out_l is None:
        out_l = torch.empty((W, B, Hq), dtype=torch.float32, device=dev)
    _need(out, torch.float32, (W, B, Hq, D), "out")
    _need(out_m, torch.float32, (W, B, Hq), "out_m")
    _need(out_l, torch.float32, (W, B, Hq), "out_l")
    c = cache._c()
    _check("paged_attn_decode_f4_noalloc",
           lib.paged_attn_decode_f4_noalloc(C.byref(c), _ptr(q), _ptr(page_table), _ptr(context_lens), B, Hq,
                                            page_table.shape[1], int(max_context_len), W, int(window_tokens),
                                            float(sm_scale), _ptr(out), _ptr(out_m), _ptr(out_l), _stream()))
    return out, out_m, out_l


def decode_rows_workspace_size(B, R, Hq, num_kv_heads, head_dim, max_context_len, num_windows=1,
                               window_tokens=0) -> int:
    return load_library().paged_attn_decode_rows_f4_workspace_size(B, R, Hq, num_kv_heads, head_dim, max_context_len,
                                                                   num_windows, window_tokens)


def paged_attn_decode_rows_f4(cache: F4Cache, q, page_table, context_lens, max_context_len: int, sm_scale: float,
                              num_windows: int = 1, window_tokens: int = 0, out=None, out_m=None, out_l=None,
                              workspace=None):
    """Decode of R query rows per sequence (q [B, R, Hq, D]; row r at position context_len - R + r);
    returns (out [W, B, R, Hq, D], m [W, B, R, Hq], l [W, B, R, Hq])."""
    lib = load_library()
    B, R, Hq, D = q.shape
    _need(q, torch.bfloat16, (B, R, Hq, D), "q")
    _need(page_table, torch.int32, None, "page_table")
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B, max_pages]")
    _need(context_lens, torch.int32, (B,), "context_lens")
    W = num_windows
    dev = q.device
    if out is None:
        out = torch.empty((W, B, R, Hq, D), dtype=torch.float32, device=dev)
    if out_m is None:
        out_m = torch.empty((W, B, R, Hq), dtype=torch.float32, device=dev)
    if out_l is None:
        out_l = torch.empty((W, B, R, Hq), dtype=torch.float32, device=dev)
    _need(out, torch.float32, (W, B, R, Hq, D), "out")
    ws_need = decode_rows_workspace_size(B, R, Hq, cache.num_kv_heads, cache.head_dim, max_context_len, W,
                                         window_tokens)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = cache._c()
    _check("paged_attn_decode_rows_f4",
           lib.paged_attn_decode_rows_f4(C.byref(c), _ptr(q), _ptr(page_table), _ptr(context_lens), B, R, Hq,
                                         page_table.shape[1], int(max_context_len), W, int(window_tokens),
                                         float(sm_scale), _ptr(out), _ptr(out_m), _ptr(out_l), _ptr(workspace),
                                         ws_bytes, _stream()))
    return out, out_m, out_l


def lse_merge(m, l, o, out=None, out_m=None, out_l=None):
    """Fold C partial states: m, l [C, R...], o [C, R..., D] -> (out [R..., D], M [R...], L [R...])."""
    lib = load_library()
    Cn = o.shape[0]
    D = o.shape[-1]
    rshape = tuple(o.shape[1:-1])
    R = math.prod(rshape)
    _need(m, torch.float32, (Cn,) + rshape, "m")
    _need(l, torch.float32, (Cn,) + rshape, "l")
    _need(o, torch.float32, None, "o")
    dev = o.device
    if out is None:
        out = torch.empty(rshape + (D,), dtype=torch.float32, device=dev)
    if out_m is None:
        out_m = torch.empty(rshape, dtype=torch.float32, device=dev)
    if out_l is None:
        out_l = torch.empty(rshape, dtype=torch.float32, device=dev)
    _check("lse_merge", lib.lse_merge(_ptr(m), _ptr(l), _ptr(o), Cn, R, D, _ptr(out), _ptr(out_m), _ptr(out_l),
                                      _stream()))
    return out, out_m, out_l


def prefill_workspace_size(T, Hq, num_kv_heads, head_dim, pos0) -> int:
    return load_library().paged_attn_prefill_f4_workspace_size(T, Hq, num_kv_heads, head_dim, pos0)


def paged_attn_prefill_f4(cache: F4Cache, q, k_new, v_new, page_table, pos0: int, sm_scale: float, out=None,
                          out_m=None, out_l=None, workspace=None):
    """Write the chunk's K/V (if given) and attend causally; returns (out [T, Hq, D], m [T, Hq], l [T, Hq])."""
    return _prefill("paged_attn_prefill_f4", cache, q, k_new, v_new, page_table, pos0, sm_scale, out, out_m, out_l,
                    workspace)


def paged_attn_prefill_f4_fp8(cache: F4Cache, q, k_new, v_new, page_table, pos0: int, sm_scale: float, out=None,
                              out_m=None, out_l=None, workspace=None):
    """paged_attn_prefill_f4 with 8-bit products (Q.K^T in INT8, P.V in E4M3); same arguments and results."""
    return _prefill("paged_attn_prefill_f4_fp8", cache, q, k_new, v_new, page_table, pos0, sm_scale, out, out_m,
                    out_l, workspace)


def _prefill(name, cache: F4Cache, q, k_new, v_new, page_table, pos0, sm_scale, out, out_m, out_l, workspace):
    lib = load_library()
    T, Hq, D = q.shape
    _need(q, torch.bfloat16, (T, Hq, D), "q")
    if k_new is not None:
        _need(k_new, torch.float32, (T, cache.num_kv_heads, cache.head_dim), "k_new")
        _need(v_new, torch.float32, (T, cache.num_kv_heads, cache.head_dim), "v_new")
    _need(page_table, torch.int32, None, "page_table")
    dev = q.device
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    if out_m is None:
        out_m = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    if out_l is None:
        out_l = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    ws_need = prefill_workspace_size(T, Hq, cache.num_kv_heads, cache.head_dim, pos0)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = cache._c()
    _check(name, getattr(lib, name)(C.byref(c), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(page_table),
                                    page_table.numel(), T, Hq, int(pos0), float(sm_scale), _ptr(out), _ptr(out_m),
                                    _ptr(out_l), _ptr(workspace), ws_bytes, _stream()))
    return out, out_m, out_l


def gather_kv_cache_f4(cache: F4Cache, page_table, cu_seq_lens, total_tokens: int, dtype=torch.bfloat16,
                       k_out=None, v_out=None):
    """Dequantise B sequences' cached K and V into rows [total_tokens, H, D] (bf16 or fp32);
    sequence b's tokens go to rows cu_seq_lens[b] .. cu_seq_lens[b + 1] - 1.  Returns (k_out, v_out)."""
    lib = load_library()
    _need(page_table, torch.int32, None, "page_table")
    if page_table.dim() != 2:
        raise ValueError("page_table must be [B, max_pages]")
    B, max_pages = page_table.shape
    _need(cu_seq_lens, torch.int32, (B + 1,), "cu_seq_lens")
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("dtype must be bfloat16 or float32")
    shape = (int(total_tokens), cache.num_kv_heads, cache.head_dim)
    dev = page_table.device
    if k_out is None:
        k_out = torch.empty(shape, dtype=dtype, device=dev)
    if v_out is None:
        v_out = torch.empty(shape, dtype=dtype, device=dev)
    _need(k_out, dtype, shape, "k_out")
    _need(v_out, dtype, shape, "v_out")
    c = cache._c()
    _check("gather_kv_cache_f4",
           lib.gather_kv_cache_f4(C.byref(c), _ptr(page_table), _ptr(cu_seq_lens), B, max_pages, int(total_tokens),
                                  _ptr(k_out), _ptr(v_out), BF16 if dtype == torch.bfloat16 else F32, _stream()))
    return k_out, v_out


class KernelTimer:
    """Times one library kernel with HIP events the library records around each
    of its launches (see f4kv_timing_start): ``with KernelTimer(KERNEL_DECODE) as t:
    ...``; afterwards ``t.total_ms``, ``t.launches`` and ``t.avg_ms``."""

    def __init__(self, kernel: int, max_launches: int = 4096):
        self.kernel, self.max_launches = kernel, max_launches
        self.total_ms, self.launches = 0.0, 0

    def __enter__(self):
        _check("f4kv_timing_start", load_library().f4kv_timing_start(self.kernel, self.max_launches))
        return self

    def __exit__(self, *exc):
        ms, n = C.c_double(0.0), C.c_int64(0)
        _check("f4kv_timing_stop", load_library().f4kv_timing_stop(self.kernel, C.byref(ms), C.byref(n)))
        self.total_ms, self.launches = ms.value, n.value
        return False

    @property
    def avg_ms(self) -> float:
        return self.total_ms / self.launches if self.launches else float("nan")


def device_checks(on: bool):
    """Switch the device-side checks of context lengths, page ids, slot ids and
    row offsets on or off (process-wide; off by default)."""
    _check("f4kv_device_checks", load_library().f4kv_device_checks(1 if on else 0))


def device_check_word() -> int:
    """Wait for the device, return the OR of the CHECK_* flags raised on the
    current device since the last read, and clear it."""
    w = C.c_uint32(0)
    _check("f4kv_device_check_word", load_library().f4kv_device_check_word(C.byref(w)))
    return int(w.value)
