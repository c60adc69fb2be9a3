// C ABI entry points: host-side validation, error state, kernel launches.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include <algorithm>

#include "f4kv_internal.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return F4KV_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(F4KV_ERR_LAUNCH, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Geometry and pointers of a cache descriptor.
int check_cache(const f4kv_cache* c, const char* fn) {
  if (!c) return fail(F4KV_ERR_INVALID, "%s: cache descriptor is NULL", fn);
  if (!c->k_nib || !c->k_scale || !c->v_nib || !c->v_scale)
    return fail(F4KV_ERR_INVALID, "%s: a cache array pointer is NULL", fn);
  if (!aligned(c->k_nib, 16) || !aligned(c->k_scale, 16) || !aligned(c->v_nib, 16) || !aligned(c->v_scale, 16))
    return fail(F4KV_ERR_INVALID, "%s: cache arrays must be 16-byte aligned", fn);
  if (c->page_size != f4kv::kPage)
    return fail(F4KV_ERR_INVALID, "%s: page_size must be 64 (got %d)", fn, c->page_size);
  if (c->v_scale_per_token != 0 && c->v_scale_per_token != 1)
    return fail(F4KV_ERR_INVALID, "%s: v_scale_per_token must be 0 or 1 (got %d)", fn, c->v_scale_per_token);
  if (c->num_pages <= 0 || c->num_kv_heads <= 0)
    return fail(F4KV_ERR_INVALID, "%s: num_pages and num_kv_heads must be positive", fn);
  if (c->num_pages > INT32_MAX / f4kv::kPage)
    return fail(F4KV_ERR_INVALID, "%s: num_pages * 64 must fit in int32 (slot ids)", fn);
  if (c->head_dim <= 0 || c->head_dim % f4kv::kBlock != 0 || c->head_dim > 4096)
    return fail(F4KV_ERR_INVALID, "%s: head_dim must be a positive multiple of 32 (<= 4096), got %d", fn,
                c->head_dim);
  const int64_t cells = static_cast<int64_t>(c->num_pages) * c->num_kv_heads * f4kv::kPage * c->head_dim;
  if (cells / 2 > (int64_t(1) << 40)) return fail(F4KV_ERR_INVALID, "%s: cache too large", fn);
  return F4KV_OK;
}

int yarn_scale(const f4kv_yarn_params* p, double* m, const char* fn) {
  if (!p) return fail(F4KV_ERR_INVALID, "%s: params is NULL", fn);
  if (!(p->theta > 1.0) || !std::isfinite(p->theta)) return fail(F4KV_ERR_INVALID, "%s: theta must be > 1", fn);
  if (p->rotary_dim <= 0 || p->rotary_dim % 2 != 0 || p->rotary_dim > 4096)
    return fail(F4KV_ERR_INVALID, "%s: rotary_dim must be even and in (0, 4096]", fn);
  if (!(p->factor == 1.0 || (p->factor > 1.0 && p->factor <= 64.0)))
    return fail(F4KV_ERR_INVALID, "%s: factor must be 1 or in (1, 64], got %g", fn, p->factor);
  if (p->factor != 1.0) {
    if (p->orig_ctx <= 0) return fail(F4KV_ERR_INVALID, "%s: orig_ctx must be positive", fn);
    if (!(p->beta_fast > p->beta_slow && p->beta_slow > 0.0) || !std::isfinite(p->beta_fast))
      return fail(F4KV_ERR_INVALID, "%s: need beta_fast > beta_slow > 0", fn);
  }
  if (!std::isfinite(p->mscale)) return fail(F4KV_ERR_INVALID, "%s: mscale is not finite", fn);
  if (p->mscale > 0.0)
    *m = p->mscale;
  else
    *m = p->factor == 1.0 ? 1.0 : 1.0 + 0.1 * std::log(p->factor);
  return F4KV_OK;
}

}  // namespace

extern "C" {

int f4kv_abi_version(void) { return F4KV_ABI_VERSION; }

const char* f4kv_last_error(void) { return g_error.c_str(); }

size_t f4kv_cache_bytes(int32_t num_pages, int32_t num_kv_heads, int32_t head_dim, int32_t v_scale_per_token,
                        size_t* k_nib, size_t* k_scale, size_t* v_nib, size_t* v_scale) {
  if (num_pages <= 0 || num_kv_heads <= 0 || head_dim <= 0 || head_dim % 32 != 0) return 0;
  if (v_scale_per_token != 0 && v_scale_per_token != 1) return 0;
  const size_t cells = static_cast<size_t>(num_pages) * num_kv_heads * f4kv::kPage;
  const size_t nib = cells * head_dim / 2;
  const size_t sc = cells * (head_dim / 32) * 2;
  const size_t vsc = v_scale_per_token ? cells * 2 : sc;
  if (k_nib) *k_nib = nib;
  if (v_nib) *v_nib = nib;
  if (k_scale) *k_scale = sc;
  if (v_scale) *v_scale = vsc;
  return 2 * nib + sc + vsc;
}

int yarn_rope_table(const f4kv_yarn_params* params, const int32_t* positions, int32_t n, float* cos_out,
                    float* sin_out, hipStream_t stream) {
  const char* fn = "yarn_rope_table";
  double m = 1.0;
  if (int r = yarn_scale(params, &m, fn)) return r;
  if (n < 0 || n > (1 << 26)) return fail(F4KV_ERR_INVALID, "%s: n out of range (%d)", fn, n);
  if (n == 0) return ok();
  if (!positions || !cos_out || !sin_out) return fail(F4KV_ERR_INVALID, "%s: NULL array", fn);
  if (!aligned(positions, 4) || !aligned(cos_out, 4) || !aligned(sin_out, 4))
    return fail(F4KV_ERR_INVALID, "%s: arrays must be 4-byte aligned", fn);
  return launched(f4kv::launch_rope_table(*params, m, positions, n, cos_out, sin_out, stream), fn);
}

int yarn_rope_apply(const float* cos_rows, const float* sin_rows, const void* x, int32_t x_dtype, void* y,
                    int32_t y_dtype, int32_t T, int32_t H, int32_t D, int32_t rotary_dim, hipStream_t stream) {
  const char* fn = "yarn_rope_apply";
  if (x_dtype != F4KV_F32 && x_dtype != F4KV_BF16) return fail(F4KV_ERR_INVALID, "%s: bad x_dtype", fn);
  if (y_dtype != F4KV_F32 && y_dtype != F4KV_BF16) return fail(F4KV_ERR_INVALID, "%s: bad y_dtype", fn);
  if (T < 0 || H < 0 || D <= 0 || D > 65536) return fail(F4KV_ERR_INVALID, "%s: bad T/H/D", fn);
  if (rotary_dim <= 0 || rotary_dim % 2 != 0 || rotary_dim > D)
    return fail(F4KV_ERR_INVALID, "%s: rotary_dim must be even and in (0, D]", fn);
  if (static_cast<int64_t>(T) * H * D > (int64_t(1) << 34)) return fail(F4KV_ERR_INVALID, "%s: too large", fn);
  if (T == 0 || H == 0) return ok();
  if (!cos_rows || !sin_rows || !x || !y) return fail(F4KV_ERR_INVALID, "%s: NULL array", fn);
  if (!aligned(x, 4) || !aligned(y, 4) || !aligned(cos_rows, 4) || !aligned(sin_rows, 4))
    return fail(F4KV_ERR_INVALID, "%s: arrays must be 4-byte aligned", fn);
  if (x == y && x_dtype != y_dtype) return fail(F4KV_ERR_INVALID, "%s: in place needs equal dtypes", fn);
  return launched(
      f4kv::launch_rope_apply(cos_rows, sin_rows, x, x_dtype, y, y_dtype, T, H, D, rotary_dim, stream), fn);
}

int kv_cache_write_f4(const f4kv_cache* cache, const float* k, const float* v, const int32_t* slot_mapping,
                      int32_t T, hipStream_t stream) {
  const char* fn = "kv_cache_write_f4";
  if (int r = check_cache(cache, fn)) return r;
  if (T < 0 || T > (1 << 26)) return fail(F4KV_ERR_INVALID, "%s: T out of range (%d)", fn, T);
  if (T == 0) return ok();
  if (!k || !v || !slot_mapping) return fail(F4KV_ERR_INVALID, "%s: NULL array", fn);
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 4))
    return fail(F4KV_ERR_INVALID, "%s: k, v must be 16-byte aligned", fn);
  if (f4kv::checks_on()) {
    hipError_t e = f4kv::check_slots(slot_mapping, T, static_cast<int64_t>(cache->num_pages) * f4kv::kPage, stream);
    if (e != hipSuccess) return launched(e, fn);
  }
  return launched(f4kv::launch_kv_write(*cache, k, v, slot_mapping, T, stream), fn);
}

size_t paged_attn_decode_f4_workspace_size(int32_t B, int32_t Hq, int32_t num_kv_heads, int32_t head_dim,
                                           int32_t max_context_len, int32_t num_windows, int32_t window_tokens) {
  return paged_attn_decode_rows_f4_workspace_size(B, 1, Hq, num_kv_heads, head_dim, max_context_len, num_windows,
                                                  window_tokens);
}

size_t paged_attn_decode_rows_f4_workspace_size(int32_t B, int32_t R, int32_t Hq, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t max_context_len, int32_t num_windows,
                                                int32_t window_tokens) {
  if (B <= 0 || R < 1 || R > 8 || Hq <= 0 || num_kv_heads <= 0 || Hq % num_kv_heads != 0 ||
      head_dim != f4kv::kHeadDim || max_context_len < 0 || num_windows <= 0 || window_tokens < 0)
    return 0;
  if (const int32_t sp = f4kv::rows_prefill_splits(B, R, Hq, num_kv_heads, max_context_len, num_windows,
                                                   window_tokens))
    return f4kv::rows_prefill_ws_bytes(B, R, Hq, sp);
  return f4kv::plan_decode(B, R, Hq, num_kv_heads, max_context_len, num_windows, window_tokens).ws_bytes;
}

}  // extern "C"

namespace {

// fixed_scratch: the workspace is the library's own device-side scratch array
// (workspace / ws_bytes are ignored); the call allocates nothing.
int decode_common(const char* fn, const f4kv_cache* cache, const uint16_t* q, const int32_t* page_table,
                  const int32_t* context_lens, int32_t B, int32_t R, int32_t Hq, int32_t max_pages,
                  int32_t max_context_len, int32_t num_windows, int32_t window_tokens, float sm_scale, float* out,
                  float* out_m, float* out_l, void* workspace, size_t ws_bytes, hipStream_t stream,
                  bool fixed_scratch = false, const f4kv::DecodeStep* step = nullptr) {
  if (int r = check_cache(cache, fn)) return r;
  const int32_t Hkv = cache->num_kv_heads;
  if (B < 0 || Hq <= 0 || max_pages <= 0 || max_context_len < 0)
    return fail(F4KV_ERR_INVALID, "%s: need B >= 0, Hq > 0, max_pages > 0, max_context_len >= 0", fn);
  if (R < 1 || R > 8) return fail(F4KV_ERR_INVALID, "%s: rows per sequence must be in [1, 8] (got %d)", fn, R);
  if (Hq % Hkv != 0) return fail(F4KV_ERR_INVALID, "%s: Hq (%d) not a multiple of num_kv_heads (%d)", fn, Hq, Hkv);
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_pages) * f4kv::kPage)
    return fail(F4KV_ERR_INVALID, "%s: max_context_len exceeds max_pages * 64", fn);
  if (num_windows <= 0 || num_windows > 65535) return fail(F4KV_ERR_INVALID, "%s: num_windows out of range", fn);
  if (window_tokens < 0 || window_tokens % f4kv::kPage != 0)
    return fail(F4KV_ERR_INVALID, "%s: window_tokens must be a non-negative multiple of 64", fn);
  if (num_windows > 1 && window_tokens == 0)
    return fail(F4KV_ERR_INVALID, "%s: several windows need window_tokens > 0", fn);
  if (!std::isfinite(sm_scale)) return fail(F4KV_ERR_INVALID, "%s: sm_scale is not finite", fn);
  if (cache->head_dim != f4kv::kHeadDim)
    return fail(F4KV_ERR_UNSUPPORTED, "%s: head_dim %d not supported (256 only)", fn, cache->head_dim);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(F4KV_ERR_UNSUPPORTED, "%s: query heads per KV head must be 1, 2, 4 or 8 (got %d)", fn, G);
  if (static_cast<int64_t>(B) * Hkv > 65535) return fail(F4KV_ERR_UNSUPPORTED, "%s: B * num_kv_heads > 65535", fn);
  if (static_cast<int64_t>(num_windows) * B * R * Hq > (int64_t(1) << 31) - 1)
    return fail(F4KV_ERR_UNSUPPORTED, "%s: too many output rows", fn);
  if (B == 0) return ok();
  if (!q || !page_table || !context_lens || !out) return fail(F4KV_ERR_INVALID, "%s: NULL array", fn);
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(page_table, 4) || !aligned(context_lens, 4) ||
      (out_m && !aligned(out_m, 4)) || (out_l && !aligned(out_l, 4)))
    return fail(F4KV_ERR_INVALID, "%s: q and out must be 16-byte aligned", fn);
  // device-side checks, once every host-side check has passed
  auto device_checks = [&]() -> hipError_t {
    if (!f4kv::checks_on()) return hipSuccess;
    hipError_t e = f4kv::check_pages(context_lens, 0, page_table, B, max_pages, max_context_len, cache->num_pages,
                                     stream);
    if (e == hipSuccess && step)
      e = f4kv::check_slots(step->slots, B, static_cast<int64_t>(cache->num_pages) * f4kv::kPage, stream);
    return e;
  };
  if (const int32_t sp = f4kv::rows_prefill_splits(B, R, Hq, Hkv, max_context_len, num_windows, window_tokens)) {
    const size_t need = f4kv::rows_prefill_ws_bytes(B, R, Hq, sp);
    if (need > 0) {
      if (!workspace || ws_bytes < need)
        return fail(F4KV_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need,
                    workspace ? ws_bytes : size_t(0));
      if (!aligned(workspace, 16)) return fail(F4KV_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
    }
    if (hipError_t e = device_checks()) return launched(e, fn);
    return launched(f4kv::launch_prefill_rows(*cache, q, page_table, context_lens, B, R, Hq, max_pages,
                                              max_context_len, sm_scale, out, out_m, out_l, workspace, sp, stream),
                    fn);
  }
  const f4kv::DecodePlan plan = f4kv::plan_decode(B, R, Hq, Hkv, max_context_len, num_windows, window_tokens);
  if (fixed_scratch) {
    if (plan.ws_bytes > f4kv::decode_scratch_bytes())
      return fail(F4KV_ERR_UNSUPPORTED,
                  "%s: this call needs %zu bytes of workspace, more than the fixed scratch of %zu bytes "
                  "(use paged_attn_decode_f4 with a workspace)",
                  fn, plan.ws_bytes, f4kv::decode_scratch_bytes());
    hipError_t e = f4kv::decode_scratch(&workspace);
    if (e != hipSuccess)
      return fail(F4KV_ERR_LAUNCH, "%s: device address of the scratch array: %s", fn, hipGetErrorString(e));
    ws_bytes = f4kv::decode_scratch_bytes();
  }
  if (plan.ws_bytes > 0) {
    if (!workspace || ws_bytes < plan.ws_bytes)
      return fail(F4KV_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, plan.ws_bytes,
                  workspace ? ws_bytes : size_t(0));
    if (!aligned(workspace, 16)) return fail(F4KV_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
  }
  if (hipError_t e = device_checks()) return launched(e, fn);
  return launched(f4kv::launch_decode(*cache, q, page_table, context_lens, B, R, Hq, max_pages, max_context_len,
                                      num_windows, window_tokens, sm_scale, out, out_m, out_l, workspace, plan,
                                      step, stream),
                  fn);
}

}  // namespace

extern "C" {

int paged_attn_decode_f4(const f4kv_cache* cache, const uint16_t* q, const int32_t* page_table,
                         const int32_t* context_lens, int32_t B, int32_t Hq, int32_t max_pages,
                         int32_t max_context_len, int32_t num_windows, int32_t window_tokens, float sm_scale,
                         float* out, float* out_m, float* out_l, void* workspace, size_t ws_bytes,
                         hipStream_t stream) {
  return decode_common("paged_attn_decode_f4", cache, q, page_table, context_lens, B, 1, Hq, max_pages,
                       max_context_len, num_windows, window_tokens, sm_scale, out, out_m, out_l, workspace, ws_bytes,
                       stream);
}

int paged_attn_decode_f4_noalloc(const f4kv_cache* cache, const uint16_t* q, const int32_t* page_table,
                                 const int32_t* context_lens, int32_t B, int32_t Hq, int32_t max_pages,
                                 int32_t max_context_len, int32_t num_windows, int32_t window_tokens, float sm_scale,
                                 float* out, float* out_m, float* out_l, hipStream_t stream) {
  return decode_common("paged_attn_decode_f4_noalloc", cache, q, page_table, context_lens, B, 1, Hq, max_pages,
                       max_context_len, num_windows, window_tokens, sm_scale, out, out_m, out_l, nullptr, 0, stream,
                       true);
}

int paged_attn_decode_step_f4(const f4kv_cache* cache, const float* cos_rows, const float* sin_rows,
                              int32_t rotary_dim, const uint16_t* q, const float* k_new, const float* v_new,
                              const int32_t* slots, const int32_t* page_table, const int32_t* context_lens,
                              int32_t B, int32_t Hq, int32_t max_pages, int32_t max_context_len, int32_t num_windows,
                              int32_t window_tokens, float sm_scale, float* out, float* out_m, float* out_l,
                              void* workspace, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "paged_attn_decode_step_f4";
  if (int r = check_cache(cache, fn)) return r;
  if (rotary_dim <= 0 || rotary_dim % 2 != 0 || rotary_dim > cache->head_dim)
    return fail(F4KV_ERR_INVALID, "%s: rotary_dim must be even and in (0, head_dim]", fn);
  if (B > 0) {
    if (!cos_rows || !sin_rows || !k_new || !v_new || !slots) return fail(F4KV_ERR_INVALID, "%s: NULL array", fn);
    if (!aligned(cos_rows, 4) || !aligned(sin_rows, 4) || !aligned(slots, 4) || !aligned(k_new, 16) ||
        !aligned(v_new, 16))
      return fail(F4KV_ERR_INVALID, "%s: k_new, v_new must be 16-byte aligned, the tables and slots 4-byte", fn);
  }
  const f4kv::DecodeStep step{cos_rows, sin_rows, rotary_dim, k_new, v_new, slots};
  return decode_common(fn, cache, q, page_table, context_lens, B, 1, Hq, max_pages, max_context_len, num_windows,
                       window_tokens, sm_scale, out, out_m, out_l, workspace, ws_bytes, stream, false, &step);
}

int paged_attn_decode_rows_f4(const f4kv_cache* cache, const uint16_t* q, const int32_t* page_table,
                              const int32_t* context_lens, int32_t B, int32_t R, int32_t Hq, int32_t max_pages,
                              int32_t max_context_len, int32_t num_windows, int32_t window_tokens, float sm_scale,
                              float* out, float* out_m, float* out_l, void* workspace, size_t ws_bytes,
                              hipStream_t stream) {
  return decode_common("paged_attn_decode_rows_f4", cache, q, page_table, context_lens, B, R, Hq, max_pages,
                       max_context_len, num_windows, window_tokens, sm_scale, out, out_m, out_l, workspace, ws_bytes,
                       stream);
}

int lse_merge(const float* m, const float* l, const float* o, int32_t C, int32_t R, int32_t D, float* out,
              float* out_m, float* out_l, hipStream_t stream) {
  const char* fn = "lse_merge";
  if (C <= 0 || R < 0 || D <= 0 || D % 4 != 0 || D > 1024)
    return fail(F4KV_ERR_INVALID, "%s: need C > 0, R >= 0, D a multiple of 4 in (0, 1024]", fn);
  if (R > (1 << 30) / 1) return fail(F4KV_ERR_INVALID, "%s: R too large", fn);
  if (R == 0) return ok();
  if (!m || !l || !o || !out) return fail(F4KV_ERR_INVALID, "%s: NULL array", fn);
  if (!aligned(o, 16) || !aligned(out, 16) || !aligned(m, 4) || !aligned(l, 4))
    return fail(F4KV_ERR_INVALID, "%s: o and out must be 16-byte aligned", fn);
  return launched(f4kv::launch_merge(m, l, o, C, R, D, out, out_m, out_l, stream), fn);
}

size_t paged_attn_prefill_f4_workspace_size(int32_t T, int32_t Hq, int32_t num_kv_heads, int32_t head_dim,
                                            int32_t pos0) {
  if (T <= 0 || Hq <= 0 || num_kv_heads <= 0 || head_dim != f4kv::kHeadDim || pos0 < 0) return 0;
  // one size for both prefill entry points
  return std::max(f4kv::plan_prefill_f16(T, Hq, num_kv_heads, pos0).ws_bytes,
                  f4kv::plan_prefill_fp8(T, Hq, num_kv_heads, pos0).ws_bytes);
}

}  // extern "C"

namespace {
// Both prefill entry points: validation, the in-call cache write, the launch.
int prefill_common(const char* fn, bool fp8, const f4kv_cache* cache, const uint16_t* q, const float* k_new,
                   const float* v_new, const int32_t* page_table, int32_t max_pages, int32_t T, int32_t Hq,
                   int32_t pos0, float sm_scale, float* out, float* out_m, float* out_l, void* workspace,
                   size_t ws_bytes, hipStream_t stream) {
  if (int r = check_cache(cache, fn)) return r;
  const int32_t Hkv = cache->num_kv_heads;
  if (T < 0 || Hq <= 0 || pos0 < 0 || max_pages <= 0)
    return fail(F4KV_ERR_INVALID, "%s: need T >= 0, Hq > 0, pos0 >= 0, max_pages > 0", fn);
  if (Hq % Hkv != 0) return fail(F4KV_ERR_INVALID, "%s: Hq not a multiple of num_kv_heads", fn);
  if (static_cast<int64_t>(pos0) + T > static_cast<int64_t>(max_pages) * f4kv::kPage)
    return fail(F4KV_ERR_INVALID, "%s: pos0 + T exceeds max_pages * 64", fn);
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(F4KV_ERR_INVALID, "%s: k_new and v_new go together", fn);
  if (!std::isfinite(sm_scale)) return fail(F4KV_ERR_INVALID, "%s: sm_scale is not finite", fn);
  if (cache->head_dim != f4kv::kHeadDim)
    return fail(F4KV_ERR_UNSUPPORTED, "%s: head_dim %d not supported (256 only)", fn, cache->head_dim);
  if (Hq / Hkv != 4) return fail(F4KV_ERR_UNSUPPORTED, "%s: 4 query heads per KV head only", fn);
  if (T > (1 << 20)) return fail(F4KV_ERR_UNSUPPORTED, "%s: T too large", fn);
  if (T == 0) return ok();
  if (!q || !page_table || !out) return fail(F4KV_ERR_INVALID, "%s: NULL array", fn);
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(page_table, 4) || (k_new && !aligned(k_new, 16)) ||
      (v_new && !aligned(v_new, 16)))
    return fail(F4KV_ERR_INVALID, "%s: q, out, k_new, v_new must be 16-byte aligned", fn);
  const f4kv::PrefillPlan plan =
      fp8 ? f4kv::plan_prefill_fp8(T, Hq, Hkv, pos0) : f4kv::plan_prefill_f16(T, Hq, Hkv, pos0);
  if (plan.ws_bytes > 0) {
    if (!workspace || ws_bytes < plan.ws_bytes)
      return fail(F4KV_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, plan.ws_bytes,
                  workspace ? ws_bytes : size_t(0));
    if (!aligned(workspace, 16)) return fail(F4KV_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
  }
  if (f4kv::checks_on()) {
    hipError_t e = f4kv::check_pages(nullptr, pos0 + T, page_table, 1, max_pages, pos0 + T, cache->num_pages, stream);
    if (e != hipSuccess) return launched(e, fn);
  }
  if (k_new) {
    hipError_t e = f4kv::launch_kv_write_paged(*cache, k_new, v_new, page_table, pos0, T, stream);
    if (e != hipSuccess) return launched(e, fn);
  }
  if (fp8)
    return launched(f4kv::launch_prefill_fp8(*cache, q, page_table, max_pages, T, Hq, pos0, sm_scale, out, out_m,
                                             out_l, workspace, plan, stream),
                    fn);
  return launched(f4kv::launch_prefill(*cache, q, page_table, max_pages, T, Hq, pos0, sm_scale, out, out_m, out_l,
                                       workspace, plan, stream),
                  fn);
}
}  // namespace

extern "C" {

int paged_attn_prefill_f4(const f4kv_cache* cache, const uint16_t* q, const float* k_new, const float* v_new,
                          const int32_t* page_table, int32_t max_pages, int32_t T, int32_t Hq, int32_t pos0,
                          float sm_scale, float* out, float* out_m, float* out_l, void* workspace,
                          size_t ws_bytes, hipStream_t stream) {
  return prefill_common("paged_attn_prefill_f4", false, cache, q, k_new, v_new, page_table, max_pages, T, Hq, pos0,
                        sm_scale, out, out_m, out_l, workspace, ws_bytes, stream);
}

int paged_attn_prefill_f4_fp8(const f4kv_cache* cache, const uint16_t* q, const float* k_new, const float* v_new,
                              const int32_t* page_table, int32_t max_pages, int32_t T, int32_t Hq, int32_t pos0,
                              float sm_scale, float* out, float* out_m, float* out_l, void* workspace,
                              size_t ws_bytes, hipStream_t stream) {
  return prefill_common("paged_attn_prefill_f4_fp8", true, cache, q, k_new, v_new, page_table, max_pages, T, Hq,
                        pos0, sm_scale, out, out_m, out_l, workspace, ws_bytes, stream);
}

int gather_kv_cache_f4(const f4kv_cache* cache, const int32_t* page_table, const int32_t* cu_seq_lens, int32_t B,
                       int32_t max_pages, int32_t total_tokens, void* k_out, void* v_out, int32_t out_dtype,
                       hipStream_t stream) {
  const char* fn = "gather_kv_cache_f4";
  if (int r = check_cache(cache, fn)) return r;
  if (out_dtype != F4KV_F32 && out_dtype != F4KV_BF16) return fail(F4KV_ERR_INVALID, "%s: bad out_dtype", fn);
  if (B < 0 || B > 65535) return fail(F4KV_ERR_INVALID, "%s: B must be in [0, 65535] (got %d)", fn, B);
  if (total_tokens < 0) return fail(F4KV_ERR_INVALID, "%s: total_tokens must be >= 0", fn);
  if (B == 0 || total_tokens == 0) return ok();
  if (max_pages <= 0 || max_pages > INT32_MAX / f4kv::kPage)
    return fail(F4KV_ERR_INVALID, "%s: max_pages out of range (%d)", fn, max_pages);
  if ((static_cast<int64_t>(max_pages) + 7) / 8 * 8 * cache->num_kv_heads > INT32_MAX)
    return fail(F4KV_ERR_INVALID, "%s: max_pages (rounded up to a multiple of 8) * num_kv_heads must fit in int32",
                fn);
  if (cache->head_dim != f4kv::kHeadDim)
    return fail(F4KV_ERR_UNSUPPORTED, "%s: head_dim %d not implemented (256 is)", fn, cache->head_dim);
  if (!page_table || !cu_seq_lens || !k_out || !v_out) return fail(F4KV_ERR_INVALID, "%s: NULL array", fn);
  if (!aligned(page_table, 4) || !aligned(cu_seq_lens, 4) || !aligned(k_out, 16) || !aligned(v_out, 16))
    return fail(F4KV_ERR_INVALID, "%s: page_table, cu_seq_lens must be 4-byte and the outputs 16-byte aligned", fn);
  if (static_cast<int64_t>(total_tokens) * cache->num_kv_heads * cache->head_dim > (int64_t(1) << 40))
    return fail(F4KV_ERR_INVALID, "%s: output too large", fn);
  if (f4kv::checks_on()) {
    hipError_t e = f4kv::check_rows(cu_seq_lens, B, page_table, max_pages, total_tokens, cache->num_pages, stream);
    if (e != hipSuccess) return launched(e, fn);
  }
  return launched(f4kv::launch_gather(*cache, page_table, cu_seq_lens, B, max_pages, total_tokens, k_out, v_out,
                                      out_dtype == F4KV_BF16, stream),
                  fn);
}

int f4kv_device_checks(int32_t on) {
  if (on != 0 && on != 1) return fail(F4KV_ERR_INVALID, "f4kv_device_checks: on must be 0 or 1 (got %d)", on);
  f4kv::set_checks(on == 1);
  return ok();
}

int f4kv_device_check_word(uint32_t* word) {
  const char* fn = "f4kv_device_check_word";
  if (!word) return fail(F4KV_ERR_INVALID, "%s: word is NULL", fn);
  hipError_t e = f4kv::read_check_word(word);
  if (e != hipSuccess) return fail(F4KV_ERR_LAUNCH, "%s: reading the device word failed: %s", fn, hipGetErrorString(e));
  return ok();
}

int f4kv_timing_start(int32_t kernel, int32_t max_launches) {
  const char* fn = "f4kv_timing_start";
  if (kernel != F4KV_KERNEL_DECODE && kernel != F4KV_KERNEL_PREFILL && kernel != F4KV_KERNEL_PREFILL_FP8)
    return fail(F4KV_ERR_INVALID, "%s: unknown kernel %d", fn, kernel);
  if (max_launches <= 0 || max_launches > (1 << 20))
    return fail(F4KV_ERR_INVALID, "%s: max_launches must be in [1, 2^20], got %d", fn, max_launches);
  hipError_t e = f4kv::timing_start(kernel, max_launches);
  if (e != hipSuccess) return fail(F4KV_ERR_LAUNCH, "%s: hipEventCreate failed: %s", fn, hipGetErrorString(e));
  return ok();
}

int f4kv_timing_stop(int32_t kernel, double* total_ms, int64_t* launches) {
  const char* fn = "f4kv_timing_stop";
  if (kernel != F4KV_KERNEL_DECODE && kernel != F4KV_KERNEL_PREFILL && kernel != F4KV_KERNEL_PREFILL_FP8)
    return fail(F4KV_ERR_INVALID, "%s: unknown kernel %d", fn, kernel);
  hipError_t e = f4kv::timing_stop(kernel, total_ms, launches);
  if (e != hipSuccess) return fail(F4KV_ERR_LAUNCH, "%s: reading the events failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // extern "C"
