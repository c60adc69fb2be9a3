// gather_kv_cache_f4: paged F4 cells -> contiguous dequantised rows.
//
// What is computed (mistral.rs PR #2375, "Changes by area" item 2: the cache's
// gather path gains an F4 variant next to the attention kernels): token i of
// sequence b becomes row cu_seq_lens[b] + i of the K and V outputs, each value
// (nibble - 8) * scale.  The product of a 4-bit code and an fp16 scale is exact
// in fp32; a bf16 output is that value rounded to nearest-even.
//
// A workgroup owns one page of one sequence and one KV head; its cells go
// through LDS so that the loads and the stores are both contiguous.  The grid
// puts the heads of a page on one XCD (their output rows interleave).
#include "f4kv_internal.h"

namespace f4kv {
namespace {

struct GatherArgs {
  const uint8_t* k_nib;
  const uint16_t* k_scale;
  const uint8_t* v_nib;
  const uint16_t* v_scale;
  const int32_t* pt;
  const int32_t* cu;
  void* k_out;
  void* v_out;
  int32_t H, num_pages, max_pages, total, bf16, v_per_token;
};

constexpr int kD = kHeadDim;  // values per head row this kernel implements

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The rows are written once and not read back by this kernel: non-temporal
// 16-byte stores (measured ~4% faster than plain ones on the 3 x 262,144-token
// bf16 gather).
template <bool BF16>
__device__ __forceinline__ void store8(void* base, int64_t elem, const float* v) {
  if (BF16) {
    u32x4 w;
    w.x = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
    w.y = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
    w.z = f32_to_bf16(v[4]) | (static_cast<uint32_t>(f32_to_bf16(v[5])) << 16);
    w.w = f32_to_bf16(v[6]) | (static_cast<uint32_t>(f32_to_bf16(v[7])) << 16);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + elem));
  } else {
    const float4_t a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
    float4_t* p = reinterpret_cast<float4_t*>(static_cast<float*>(base) + elem);
    __builtin_nontemporal_store(a, p);
    __builtin_nontemporal_store(b, p + 1);
  }
}

// 8 consecutive nibbles of x (low first) as (n - 8) * sc.
__device__ __forceinline__ void dequant8(uint32_t x, float sc, float* v) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = static_cast<float>(static_cast<int>((x >> (4 * e)) & 15u) - 8) * sc;
}

// 16 bytes with the non-temporal hint (the line is not kept for reuse).
__device__ __forceinline__ uint4 nt_load(const uint4* p) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

template <bool BF16>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  // blockIdx.x = (page / 8 * H + head) * 8 + page % 8: the workgroups are
  // dealt to the XCDs in turn, so the H heads of a page (whose output rows
  // interleave) run on one XCD, and consecutive pages on different ones.
  const int x8 = blockIdx.x & 7, rest = static_cast<int>(blockIdx.x >> 3);
  const int h = rest % a.H, lp = (rest / a.H) * 8 + x8, b = blockIdx.y;
  if (lp >= a.max_pages) return;
  const int tid = threadIdx.x;
  const int32_t row0 = a.cu[b];
  const int32_t len = a.cu[b + 1] - row0;
  if (len <= 0 || lp * kPage >= len) return;  // uniform over the workgroup
  const int32_t pid = a.pt[static_cast<int64_t>(b) * a.max_pages + lp];
  const bool valid = static_cast<uint32_t>(pid) < static_cast<uint32_t>(a.num_pages);
  const int64_t ph = static_cast<int64_t>(valid ? pid : 0) * a.H + h;
  constexpr int nb = kD / kBlock;

  // The page's K units (block c, token t), V units (token group c, channel
  // quad j) and scales are staged in LDS with coalesced 16-byte loads; then
  // each thread writes 8 consecutive channels of one row, 32 threads a whole
  // row, so every store instruction of a wave writes two contiguous rows.
  __shared__ uint4 kt[nb][kPage];
  __shared__ uint4 vt[kPage / 8][kD / 4];
  __shared__ uint16_t ks[kPage][nb];
  __shared__ uint16_t vs[kPage][nb];
  const uint4 zero = make_uint4(0, 0, 0, 0);
  // (non-temporal loads: each cell is read once)
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int u = tid + 256 * s;
    (&kt[0][0])[u] = valid ? nt_load(reinterpret_cast<const uint4*>(a.k_nib) + ph * (nb * kPage) + u) : zero;
    (&vt[0][0])[u] = valid ? nt_load(reinterpret_cast<const uint4*>(a.v_nib) + ph * (kPage / 8 * kD / 4) + u) : zero;
  }
  for (int i = tid; i < kPage * nb; i += 256) {
    (&ks[0][0])[i] = valid ? __builtin_nontemporal_load(a.k_scale + ph * kPage * nb + i) : 0;
    if (!a.v_per_token) (&vs[0][0])[i] = valid ? __builtin_nontemporal_load(a.v_scale + ph * kPage * nb + i) : 0;
  }
  if (a.v_per_token && tid < kPage) vs[tid][0] = valid ? __builtin_nontemporal_load(a.v_scale + ph * kPage + tid) : 0;
  __syncthreads();

  const int l = tid & 31;  // channels 8l .. 8l + 7: block l / 4
  const int c = l >> 2, d = l & 3;
#pragma unroll
  for (int it = 0; it < kPage / 8; ++it) {
    const int t = 8 * it + (tid >> 5);
    const int32_t i = lp * kPage + t;
    const int64_t row = static_cast<int64_t>(row0) + i;
    if (i >= len || row < 0 || row >= a.total) continue;  // rows outside [0, total) are never written
    const int64_t e0 = (row * a.H + h) * kD + 8 * l;
    float v[8];
    // K: dword d of unit (c, t) holds elements 8d .. 8d + 7 of block c
    const uint4 kw = kt[c][t];
    dequant8(d == 0 ? kw.x : d == 1 ? kw.y : d == 2 ? kw.z : kw.w, f16bits_to_f32(ks[t][c]), v);
    store8<BF16>(a.k_out, e0, v);
    // V: units (t / 8, 2l) and (t / 8, 2l + 1); byte 4k + 2r (+1) of a unit holds
    // its channels 0-1 (2-3) of token 8 (t / 8) + 2k + r
    const int k = (t & 7) >> 1, r = t & 1;
    const uint4 u0 = vt[t >> 3][2 * l], u1 = vt[t >> 3][2 * l + 1];
    const uint32_t w0 = k == 0 ? u0.x : k == 1 ? u0.y : k == 2 ? u0.z : u0.w;
    const uint32_t w1 = k == 0 ? u1.x : k == 1 ? u1.y : k == 2 ? u1.z : u1.w;
    const uint32_t n = ((w0 >> (16 * r)) & 0xFFFFu) | (((w1 >> (16 * r)) & 0xFFFFu) << 16);
    dequant8(n, f16bits_to_f32(a.v_per_token ? vs[t][0] : vs[t][c]), v);
    store8<BF16>(a.v_out, e0, v);
  }
}

}  // namespace

hipError_t launch_gather(const f4kv_cache& c, const int32_t* pt, const int32_t* cu, int32_t B, int32_t max_pages,
                         int32_t total, void* k_out, void* v_out, bool bf16, hipStream_t s) {
  if (B == 0 || total == 0) return hipSuccess;
  GatherArgs a;
  a.k_nib = c.k_nib;
  a.k_scale = c.k_scale;
  a.v_nib = c.v_nib;
  a.v_scale = c.v_scale;
  a.pt = pt;
  a.cu = cu;
  a.k_out = k_out;
  a.v_out = v_out;
  a.H = c.num_kv_heads;
  a.num_pages = c.num_pages;
  a.max_pages = max_pages;
  a.total = total;
  a.bf16 = bf16;
  a.v_per_token = c.v_scale_per_token;
  const dim3 grid((max_pages + 7) / 8 * 8 * c.num_kv_heads, B);  // both checked by the caller
  if (bf16)
    hipLaunchKernelGGL(gather_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(gather_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace f4kv
