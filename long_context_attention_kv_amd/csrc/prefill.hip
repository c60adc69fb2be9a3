// paged_attn_prefill_f4: causal attention of a prompt chunk over the F4 cache.
//
// What is computed (ignis context-and-speculation, --model-prefill-chunk row:
// prompts are processed in chunks; FreeToken issue #568, "Proposed solution"
// item 2: a prefill attends within a device window; mistral.rs PR #2375,
// "Changes by area" item 2: F4 cells are dequantised inside attention): query
// row i of the chunk, at position pos0 + i, attends to cache tokens
// [0, pos0 + i] after the chunk's own keys and values were written.
//
// Shape of the work.  A workgroup (4 waves) owns 32 consecutive query
// positions of one KV head, i.e. 128 query rows once the 4 query heads of the
// group are stacked (32 per wave), and a range of key pages.  Per page of 64 keys:
//  1. the workgroup dequantises the page's K and V cells into LDS as fp16,
//     K as [token][channel] and V transposed as [channel][token], each as an
//     fp16 pair hi + lo (hi = fp16(x), lo = fp16(x - hi)): a single fp16
//     rounding of the dequantised keys alone moves the output by up to ~2e-3
//     of its RMS, and of V or P by ~1e-3 each;
//  2. each wave forms S^T = K Q^T for its 32 query rows with fp16 MFMA
//     (v_mfma_f32_32x32x16_f16, fp32 accumulate) as K_hi Q + K_lo Q, so one
//     lane owns one query row and its row max / sum are mostly lane-local;
//  3. online softmax in log2 units;
//  4. O^T += V^T P^T with the same MFMA as V_hi P_hi + V_lo P_hi + V_hi P_lo,
//     P split into fp16 hi + lo like V, so only K's fp16 rounding remains.
//     The exp'd scores already sit in the B-operand lanes; the token order
//     inside a k-step is permuted to match and the V^T reads use the same
//     permutation.
// Queries keep their 64 fp16 operand registers for the whole loop.  Longer
// key ranges are split over several workgroups and folded by the merge kernel.
#include "f4kv_internal.h"

namespace f4kv {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kCT = 1;             // 32-row column tiles per wave
constexpr int kQPos = kWaves * kCT * 8;  // query positions per workgroup
constexpr int kG = 4;              // query heads per KV head
constexpr int kKStride = kHeadDim + 8;   // fp16 per K row in LDS (528 B)
constexpr int kVStride = kPage + 8;      // fp16 per V^T row in LDS (144 B, 16-byte aligned rows)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct PrefillArgs {
  const uint8_t* k_nib;
  const uint16_t* k_scale;
  const uint8_t* v_nib;
  const uint16_t* v_scale;
  const uint16_t* q;
  const int32_t* pt;
  float* o;  // [S][R][D], R = T * Hq
  float* m;  // [S][R] or null
  float* l;
  int32_t T, Hq, Hkv, num_pages, max_pages, pos0;
  int32_t kv_splits;
  float qk_scale;  // sm_scale * log2(e)
};

struct __align__(16) PrefillSmem {
  _Float16 k[2][kPage][kKStride];      // K as hi, lo * 2^10
  _Float16 vt[2][kHeadDim][kVStride];  // V^T as hi, lo
};

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a) {
  __shared__ PrefillSmem sm;
  const int qt = blockIdx.x;     // query tile
  const int g = blockIdx.y;      // KV head
  const int split = blockIdx.z;  // key-range split
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;

  // column tile c of this wave: positions (wave*kCT + c)*8 + col/4, head col % 4
  int qi[kCT], qpos[kCT];
  bool qvalid[kCT];
  const int hq = g * kG + (col & 3);
#pragma unroll
  for (int c = 0; c < kCT; ++c) {
    qi[c] = qt * kQPos + (wave * kCT + c) * 8 + col / 4;
    qvalid[c] = qi[c] < a.T;
    qpos[c] = a.pos0 + qi[c];
  }

  // key pages this workgroup covers: up to the tile's last position, split evenly
  const int tile_last = min(a.T, (qt + 1) * kQPos) - 1;
  const int npages = (a.pos0 + tile_last) / kPage + 1;
  const int per = (npages + a.kv_splits - 1) / a.kv_splits;
  const int pbeg = split * per;
  const int pend = min(npages, pbeg + per);

  // Q^T operands: lane holds q[row][16 s + 8 half + 0..7] for s = 0..15
  half8_t qf[kCT][16];
#pragma unroll
  for (int c = 0; c < kCT; ++c) {
    const uint16_t* qrow = a.q + (static_cast<int64_t>(qvalid[c] ? qi[c] : 0) * a.Hq + hq) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * half);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = word(raw, j);
        qf[c][s][2 * j] = static_cast<_Float16>(bf16_to_f32(static_cast<uint16_t>(w)));
        qf[c][s][2 * j + 1] = static_cast<_Float16>(bf16_to_f32(static_cast<uint16_t>(w >> 16)));
      }
    }
  }

  float16_t acc[kCT][8];  // O^T per column tile: 8 channel tiles of 32
#pragma unroll
  for (int c = 0; c < kCT; ++c)
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[c][d] = float16_t{};
  float m_run[kCT], l_lane[kCT];
#pragma unroll
  for (int c = 0; c < kCT; ++c) {
    m_run[c] = -INFINITY;
    l_lane[c] = 0.0f;
  }

  for (int lp = pbeg; lp < pend; ++lp) {
    int32_t pid = a.pt[lp];
    const bool pvalid = static_cast<uint32_t>(pid) < static_cast<uint32_t>(a.num_pages);
    pid = pvalid ? pid : 0;
    const int64_t ph = static_cast<int64_t>(pid) * a.Hkv + g;
    const uint4* ktile = reinterpret_cast<const uint4*>(a.k_nib + ph * (kPage * kHeadDim / 2));
    const uint4* vtile = reinterpret_cast<const uint4*>(a.v_nib + ph * (kPage * kHeadDim / 2));
    uint4 kraw[2], vraw[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      kraw[r] = ktile[tid + r * kThreads];
      vraw[r] = vtile[tid + r * kThreads];
    }
    __syncthreads();  // previous page's LDS reads are done
    // ---- dequantise K: units (block c, token t) of 16 bytes ----
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int u = tid + r * kThreads;
      const int c = u >> 6, t = u & 63;
      const float s = static_cast<float>(__builtin_bit_cast(_Float16, a.k_scale[(ph * kPage + t) * 8 + c]));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = word(kraw[r], j);
        half8_t v8, l8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = static_cast<float>(static_cast<int>((w >> (4 * e)) & 0xFu) - 8) * s;  // exact
          const _Float16 hi = static_cast<_Float16>(x);
          v8[e] = hi;
          l8[e] = static_cast<_Float16>((x - static_cast<float>(hi)) * 1024.0f);
        }
        *reinterpret_cast<half8_t*>(&sm.k[0][t][32 * c + 8 * j]) = v8;
        *reinterpret_cast<half8_t*>(&sm.k[1][t][32 * c + 8 * j]) = l8;
      }
    }
    // ---- dequantise V: units (c, j) = tokens 8c..8c+7 x channels 4j..4j+3 ----
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int u = tid + r * kThreads;
      const int c = u >> 6, j = u & 63;
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        half8_t v8, l8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {  // token 8c + e sits in dword e/2, half e%2
          const int t = 8 * c + e;
          const uint32_t w = word(vraw[r], e >> 1);
          const int n = static_cast<int>((w >> (16 * (e & 1) + 4 * dd)) & 0xFu) - 8;
          const float s = static_cast<float>(__builtin_bit_cast(_Float16, a.v_scale[(ph * kPage + t) * 8 + (j >> 3)]));
          const float x = static_cast<float>(n) * s;  // exact in fp32
          const _Float16 hi = static_cast<_Float16>(x);
          v8[e] = hi;
          l8[e] = static_cast<_Float16>((x - static_cast<float>(hi)) * 1024.0f);
        }
        *reinterpret_cast<half8_t*>(&sm.vt[0][4 * j + dd][8 * c]) = v8;
        *reinterpret_cast<half8_t*>(&sm.vt[1][4 * j + dd][8 * c]) = l8;
      }
    }
    __syncthreads();

    // ---- per 32-token tile: S^T = K Q^T, online softmax, O^T += V^T P^T ----
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float16_t st[kCT], sl[kCT];
#pragma unroll
      for (int c = 0; c < kCT; ++c) {
        st[c] = float16_t{};
        sl[c] = float16_t{};
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        if ((s & 3) == 0) __builtin_amdgcn_sched_barrier(0);  // bound the K operand reads in flight
        const half8_t ka = *reinterpret_cast<const half8_t*>(&sm.k[0][tt * 32 + col][16 * s + 8 * half]);
        const half8_t kl = *reinterpret_cast<const half8_t*>(&sm.k[1][tt * 32 + col][16 * s + 8 * half]);
#pragma unroll
        for (int c = 0; c < kCT; ++c) {
          st[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[c][s], st[c], 0, 0, 0);
          sl[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kl, qf[c][s], sl[c], 0, 0, 0);
        }
      }
#pragma unroll
      for (int c = 0; c < kCT; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[c][i] = fmaf(sl[c][i], 1.0f / 1024.0f, st[c][i]);
      // B operands per [column tile][k-step of this token tile]: P * 2^15 as hi and lo
      // (for V hi), and P * 2^5 (for V lo, which LDS holds times 2^10).  The power-of-two
      // offsets keep every fp16 operand out of the subnormal range; the accumulator
      // carries P * 2^15 throughout and the epilogue divides it out.
      half8_t pb[kCT][2], pl[kCT][2], pv5[kCT][2];
#pragma unroll
      for (int c = 0; c < kCT; ++c) {
        // scores of this lane's query row (log2 units), causal mask
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tok = lp * kPage + tt * 32 + (i / 4) * 8 + half * 4 + (i % 4);
          const bool ok = pvalid && qvalid[c] && tok <= qpos[c];
          st[c][i] = ok ? st[c][i] * a.qk_scale : -INFINITY;
          mx = fmaxf(mx, st[c][i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m_run[c], mx);
        const float ms = mn == -INFINITY ? 0.0f : mn;
        const float alpha = __builtin_amdgcn_exp2f(m_run[c] - ms);
        m_run[c] = mn;
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(st[c][i] - ms);
          psum += pv;
          const float ps = pv * 32768.0f;
          const _Float16 ph = static_cast<_Float16>(ps);
          pb[c][i / 8][i % 8] = ph;
          pl[c][i / 8][i % 8] = static_cast<_Float16>(ps - static_cast<float>(ph));
          pv5[c][i / 8][i % 8] = static_cast<_Float16>(pv * 32.0f);
        }
        l_lane[c] = fmaf(l_lane[c], alpha, psum);
        if (__ballot(alpha != 1.0f)) {  // rescale only when some row's max moved
#pragma unroll
          for (int d = 0; d < 8; ++d) acc[c][d] *= alpha;
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        // k-step covers tokens base + {0..3, 8..11} (+4 for the upper half lanes)
        const int base = tt * 32 + s2 * 16 + 4 * half;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          __builtin_amdgcn_sched_barrier(0);  // bound the V^T operand reads in flight
#pragma unroll
          for (int part = 0; part < 2; ++part) {
            const _Float16* vrow = &sm.vt[part][d * 32 + col][0];
            const half4_t a0 = *reinterpret_cast<const half4_t*>(vrow + base);
            const half4_t a1 = *reinterpret_cast<const half4_t*>(vrow + base + 8);
            half8_t va;
            va[0] = a0[0]; va[1] = a0[1]; va[2] = a0[2]; va[3] = a0[3];
            va[4] = a1[0]; va[5] = a1[1]; va[6] = a1[2]; va[7] = a1[3];
#pragma unroll
            for (int c = 0; c < kCT; ++c) {
              if (part == 0) {  // V hi x (P hi + P lo); P lo x V lo is below fp32 rounding
                acc[c][d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[c][s2], acc[c][d], 0, 0, 0);
                acc[c][d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pl[c][s2], acc[c][d], 0, 0, 0);
              } else {          // (V lo * 2^10) x (P * 2^5)
                acc[c][d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pv5[c][s2], acc[c][d], 0, 0, 0);
              }
            }
          }
        }
      }
    }
  }

  // ---- epilogue: this lane's two query rows ----
  const int R = a.T * a.Hq;
#pragma unroll
  for (int c = 0; c < kCT; ++c) {
    const float L = l_lane[c] + __shfl_xor(l_lane[c], 32, 64);
    if (!qvalid[c]) continue;
    const int64_t row = static_cast<int64_t>(split) * R + static_cast<int64_t>(qi[c]) * a.Hq + hq;
    const float inv = L > 0.0f ? 1.0f / (L * 32768.0f) : 0.0f;  // P was carried times 2^15
    float* dst = a.o + row * kHeadDim;
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float4_t v;
        v.x = acc[c][d][4 * i4 + 0] * inv;
        v.y = acc[c][d][4 * i4 + 1] * inv;
        v.z = acc[c][d][4 * i4 + 2] * inv;
        v.w = acc[c][d][4 * i4 + 3] * inv;
        *reinterpret_cast<float4_t*>(dst + d * 32 + i4 * 8 + half * 4) = v;
      }
    if (half == 0) {
      if (a.m) a.m[row] = L > 0.0f ? m_run[c] * kLn2 : -INFINITY;
      if (a.l) a.l[row] = L;
    }
  }
}

}  // namespace

PrefillPlan plan_prefill(int32_t T, int32_t Hq, int32_t Hkv, int32_t pos0) {
  PrefillPlan p;
  p.q_tiles = (T + kQPos - 1) / kQPos;
  const int64_t total_pages = (static_cast<int64_t>(pos0) + T + kPage - 1) / kPage;
  // enough workgroups to cover the chip twice over when the key range is long
  const int64_t wgs = static_cast<int64_t>(p.q_tiles) * Hkv;
  int64_t splits = (512 + wgs - 1) / std::max<int64_t>(wgs, 1);
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, total_pages / 16));
  p.kv_splits = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(splits, 16)));
  const int64_t R = static_cast<int64_t>(T) * Hq;
  p.ws_bytes = p.kv_splits > 1 ? static_cast<size_t>(p.kv_splits) * R * (kHeadDim + 2) * sizeof(float) : 0;
  return p;
}

hipError_t launch_prefill(const f4kv_cache& c, const uint16_t* q, const int32_t* pt, int32_t max_pages,
                          int32_t T, int32_t Hq, int32_t pos0, float sm_scale, float* out, float* out_m,
                          float* out_l, void* ws, const PrefillPlan& plan, hipStream_t s) {
  if (T == 0) return hipSuccess;
  PrefillArgs a;
  a.k_nib = c.k_nib;
  a.k_scale = c.k_scale;
  a.v_nib = c.v_nib;
  a.v_scale = c.v_scale;
  a.q = q;
  a.pt = pt;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = c.num_kv_heads;
  a.num_pages = c.num_pages;
  a.max_pages = max_pages;
  a.pos0 = pos0;
  a.kv_splits = plan.kv_splits;
  a.qk_scale = sm_scale * kLog2e;
  const int64_t R = static_cast<int64_t>(T) * Hq;
  float* pm = nullptr;
  float* pl = nullptr;
  if (plan.kv_splits > 1) {
    float* base = static_cast<float*>(ws);
    a.o = base;
    pm = base + static_cast<size_t>(plan.kv_splits) * R * kHeadDim;
    pl = pm + static_cast<size_t>(plan.kv_splits) * R;
    a.m = pm;
    a.l = pl;
  } else {
    a.o = out;
    a.m = out_m;
    a.l = out_l;
  }
  timing_begin(F4KV_KERNEL_PREFILL, s);
  hipLaunchKernelGGL(prefill_kernel, dim3(plan.q_tiles, a.Hkv, plan.kv_splits), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  timing_end(F4KV_KERNEL_PREFILL, s);
  if (e != hipSuccess || plan.kv_splits == 1) return e;
  return launch_merge(pm, pl, a.o, plan.kv_splits, static_cast<int32_t>(R), kHeadDim, out, out_m, out_l, s);
}

}  // namespace f4kv
