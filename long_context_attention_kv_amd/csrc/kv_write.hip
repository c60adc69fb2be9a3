// kv_cache_write_f4: fp32 keys/values -> paged F4 cells.
//
// Format from mistral.rs PR #2375 ("Changes by area" item 2): symmetric 4-bit
// values (nibble - 8) * scale, 32 values per 16-byte row; error bound max_abs/16
// ("Known limitations").  The scale is fp16(absmax / 8), nearest-even, saturated
// at 65504; codes round x / s to nearest-even and clamp to [-8, 7].
//
// Exact rounding decisions: x is fp32 and s is fp16, so an inexact x / s lies at
// least 2^-24 |x / s| away from any half-integer.  The quotient is therefore
// formed in fp64 (correctly rounded, error <= 2^-53 relative), which decides
// every tie and near-tie exactly; an fp32 quotient could land on a false tie.
//
// One thread owns one 32-value block of one token's K or V row: it writes the
// block's 16 bytes (K) or eight 2-byte pieces (V) and its scale, so no byte is
// shared between threads.  When V carries one scale per token and head (the
// per-token V scale of the same item), each V thread takes the absmax of the
// token's whole V row (the 8 threads of a row read it each; the
// writer is not on the decode clock), quantises its own block against that
// scale, and the thread of block 0 writes the scale.
#include "f4kv_device.h"

namespace f4kv {
namespace {

struct KvWriteArgs {
  uint8_t* k_nib;
  uint16_t* k_scale;
  uint8_t* v_nib;
  uint16_t* v_scale;
  const float* k;
  const float* v;
  const int32_t* slots;      // slot per token, or null: use page_table and pos0
  const int32_t* page_table;
  int32_t pos0;
  int64_t per_kind;  // T * H * (D / 32)
  int32_t H, D, num_pages;
  int32_t v_per_token;  // V scale per (token, head) instead of per 32 values
};

__global__ __launch_bounds__(256) void kv_write_kernel(KvWriteArgs a) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= 2 * a.per_kind) return;
  const int kind = gid >= a.per_kind ? 1 : 0;  // 0 = K, 1 = V
  const int64_t r = kind ? gid - a.per_kind : gid;
  const int nb = a.D / kBlock;
  const int c = static_cast<int>(r % nb);
  const int64_t th = r / nb;
  const int h = static_cast<int>(th % a.H);
  const int64_t t = th / a.H;

  int32_t slot;
  if (a.slots) {
    slot = a.slots[t];
  } else {
    const int64_t pos = a.pos0 + t;
    const int32_t pg = a.page_table[pos / kPage];
    // out-of-range page ids (negative or >= num_pages) write nothing; the
    // compare comes before the multiply, which would overflow for ids >= 2^25
    if (static_cast<uint32_t>(pg) >= static_cast<uint32_t>(a.num_pages)) return;
    slot = pg * kPage + static_cast<int32_t>(pos % kPage);
  }
  if (slot < 0 || slot >= static_cast<int64_t>(a.num_pages) * kPage) return;
  const int page = slot / kPage;
  const int off = slot % kPage;

  const float4_t* src = reinterpret_cast<const float4_t*>(
      (kind ? a.v : a.k) + (t * a.H + h) * a.D + c * kBlock);
  float x[kBlock];
#pragma unroll
  for (int i = 0; i < kBlock / 4; ++i) {
    float4_t f = src[i];
    x[4 * i + 0] = f.x;
    x[4 * i + 1] = f.y;
    x[4 * i + 2] = f.z;
    x[4 * i + 3] = f.w;
  }
  float amax = 0.0f;
  if (kind == 1 && a.v_per_token) {
    const float4_t* row = reinterpret_cast<const float4_t*>(a.v + (t * a.H + h) * a.D);
    for (int i = 0; i < a.D / 4; ++i) {
      const float4_t f = row[i];
      amax = fmaxf(fmaxf(amax, fabsf(f.x)), fmaxf(fabsf(f.y), fmaxf(fabsf(f.z), fabsf(f.w))));
    }
  } else {
#pragma unroll
    for (int i = 0; i < kBlock; ++i) amax = fmaxf(amax, fabsf(x[i]));
  }

  uint32_t nib[kBlock];
  const uint16_t sbits = f4_quantize_block(x, amax, nib);
  const int64_t ph = static_cast<int64_t>(page) * a.H + h;
  if (kind == 0)
    f4_store_k_block(a.k_nib, a.k_scale, ph, nb, c, off, nib, sbits);
  else
    f4_store_v_block(a.v_nib, a.v_scale, ph, a.D, c, off, nib, sbits, a.v_per_token != 0);
}

}  // namespace

namespace {
hipError_t launch_common(const f4kv_cache& c, const float* k, const float* v, const int32_t* slots,
                         const int32_t* page_table, int32_t pos0, int32_t T, hipStream_t s) {
  if (T == 0) return hipSuccess;
  KvWriteArgs a;
  a.page_table = page_table;
  a.pos0 = pos0;
  a.k_nib = c.k_nib;
  a.k_scale = c.k_scale;
  a.v_nib = c.v_nib;
  a.v_scale = c.v_scale;
  a.k = k;
  a.v = v;
  a.slots = slots;
  a.H = c.num_kv_heads;
  a.D = c.head_dim;
  a.num_pages = c.num_pages;
  a.v_per_token = c.v_scale_per_token;
  a.per_kind = static_cast<int64_t>(T) * a.H * (a.D / kBlock);
  const int64_t total = 2 * a.per_kind;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(kv_write_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, s, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_kv_write(const f4kv_cache& c, const float* k, const float* v, const int32_t* slots, int32_t T,
                           hipStream_t s) {
  return launch_common(c, k, v, slots, nullptr, 0, T, s);
}

hipError_t launch_kv_write_paged(const f4kv_cache& c, const float* k, const float* v, const int32_t* page_table,
                                 int32_t pos0, int32_t T, hipStream_t s) {
  return launch_common(c, k, v, nullptr, page_table, pos0, T, s);
}

}  // namespace f4kv
