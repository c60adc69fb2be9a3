// paged_attn_decode_f4: split-K paged GQA decode over the F4 cache.
//
// What is computed (mistral.rs PR #2375, "Changes by area" item 2: the paged
// attention kernels read the packed F4 cells and dequantise them inline;
// FreeToken issue #568, "Proposed solution" item 2: windows folded by
// log2-sum-exp): for each (window, sequence, query head) the exact softmax
// attention of one query row over the window's cached tokens, returned as the
// partial state (m, l, o).
//
// Work split.  A workgroup of 4 waves owns a run of pages of one (window,
// sequence, KV head); each wave streams every 4th page of the run with its own
// running max / sum / output, the waves fold in LDS at the end, and the
// workgroups of one window are folded by the merge kernel.
//
// Per page (64 tokens) a wave does two phases:
//  * keys: lane = token.  The lane loads its token's 8 blocks (8 x 16 B, each
//    load instruction of the wave reads 1 KB contiguous thanks to the
//    block-major K tile) and forms the G logits with packed fp16 dot products.
//    A nibble n is turned into an fp16 operand with one AND: 0x000F000F picks
//    two nibbles into the mantissas of an fp16 pair, i.e. the subnormals
//    n * 2^-24; 0x00F000F0 picks the next two as 16 n * 2^-24 (the matching
//    query pair is pre-divided by 16).  The "- 8" of (n - 8) * s is folded into
//    the accumulator's start value (-8 * 2^-24 * sum of the block's query
//    values), and the block scale is applied once per block.
//  * values: lane = 4 consecutive channels.  The V tile stores 8 tokens x 4
//    channels per 16-byte unit, two tokens per dword, so the same AND trick
//    yields fp16 pairs over two tokens and a dot product accumulates
//    p_t s_t (n_t - 8) over token pairs.  The weights w = p_t * s_t (softmax
//    weight times the token's block scale) travel from the key phase to the
//    value phase through LDS as an fp16 pair hi + lo (hi = fp16(w), lo =
//    fp16(w - hi)), and each product is taken twice, once per part: a single
//    fp16 weight (11 bits) leaves ~2e-3 of the output RMS on channels whose
//    values are many times the others' (outlier channels), the split keeps
//    ~22 bits.  The "- 8" is corrected once per page with the page's summed
//    weights.
// The query is pre-scaled by a power of two per head so its fp16 copy keeps
// full precision whatever its magnitude; fp32 accumulation throughout.
#include <atomic>

#include "f4kv_internal.h"

namespace f4kv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kWRow = 68;  // fp32 weights per (head, block) row: 64 tokens + 16 B pad
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Query operands of one (sequence, KV head), prepared once per call and read by
// the decode kernel with scalar loads (the same for every lane).
template <int G>
struct __align__(64) QPrep {
  uint32_t pair[G][8][4][4];  // fp16 pairs [head][block][dword][pair], scaled by 2^e_h
  float qinit[G][8];          // -8 * 2^-24 * sum of the block's scaled query values
  float kscale[G];            // 2^(24 - e_h) * sm_scale * log2(e)
};

struct DecodeArgs {
  const uint8_t* k_nib;
  const uint16_t* k_scale;
  const uint8_t* v_nib;
  const uint16_t* v_scale;
  const uint16_t* q;
  const int32_t* pt;
  const int32_t* ctx;
  float* o;  // [S][R][D]
  float* m;  // [S][R] or null
  float* l;  // [S][R] or null
  int32_t B, Hq, Hkv, num_pages, max_pages, max_ctx;
  int32_t window_tokens, pages_per_split;
  float qk_scale;  // sm_scale * log2(e)
};

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

// DPP lane permutations within a row of 16 lanes (gfx9 encodings).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each half row
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within each row

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF,
                                                               false));
}

// Max over the 64 lanes, returned in every lane: DPP within rows of 16, then
// the four row results read into scalars.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  x = fmaxf(x, dpp<kDppMirror>(x));
  const int xi = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Sum over each group of 8 consecutive lanes, returned in all 8.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ float f16_lo(uint32_t w) { return f16bits_to_f32(static_cast<uint16_t>(w)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return f16bits_to_f32(static_cast<uint16_t>(w >> 16)); }

// Makes a loaded value opaque at this point so the compiler cannot start its
// unpacking any earlier (it otherwise unpacks every block right after the
// loads and spills the result).
__device__ __forceinline__ void pin(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

__device__ __forceinline__ void lds_wave_sync() {
  // LDS writes of other lanes of this wave must land before it reads them
  // (LDS executes one wave's instructions in order; this keeps the compiler
  // from moving the reads above the writes).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One workgroup per (sequence, KV head): query rows -> QPrep.
template <int G>
__global__ __launch_bounds__(kThreads) void decode_qprep_kernel(const uint16_t* __restrict__ q,
                                                               QPrep<G>* __restrict__ out, int32_t Hq,
                                                               int32_t Hkv, float qk_scale) {
  __shared__ float qf[G][kHeadDim];
  __shared__ int32_t qexp[G];
  const int b = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  QPrep<G>& P = out[blockIdx.x];
  const uint16_t* qsrc = q + (static_cast<int64_t>(b) * Hq + g * G) * kHeadDim;
  for (int i = tid; i < G * kHeadDim; i += kThreads) qf[i / kHeadDim][i % kHeadDim] = bf16_to_f32(qsrc[i]);
  __syncthreads();
  for (int h = wave; h < G; h += kWaves) {
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) mx = fmaxf(mx, fabsf(qf[h][lane + 64 * k]));
    mx = wave_max(mx);
    if (lane == 0) {
      int e = 0;
      if (mx > 0.0f) {
        int ex;
        frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
        e = 11 - ex;      // scaled max in [2^10, 2^11)
      }
      qexp[h] = e;
      P.kscale[h] = ldexpf(qk_scale, 24 - e);
    }
  }
  __syncthreads();
  for (int i = tid; i < G * 128; i += kThreads) {
    const int h = i / 128, r = i % 128;
    const int c = r / 16, k = (r / 4) % 4, p = r % 4;
    // pair p of dword k holds channels (base + p, base + p + 4); odd p are the x16 slots
    const int base = 32 * c + 8 * k + p;
    const float sc = ldexpf((p & 1) ? 0.0625f : 1.0f, qexp[h]);
    const _Float16 lo = static_cast<_Float16>(qf[h][base] * sc);
    const _Float16 hi = static_cast<_Float16>(qf[h][base + 4] * sc);
    P.pair[h][c][k][p] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
  }
  for (int i = tid; i < G * 8; i += kThreads) {
    const int h = i / 8, c = i % 8;
    float sum = 0.0f;
    for (int d = 0; d < kBlock; ++d) {
      const float v = qf[h][32 * c + d];
      // the value each channel contributes through its fp16 operand
      const float rep = (d & 1) ? 16.0f * static_cast<float>(static_cast<_Float16>(v * ldexpf(0.0625f, qexp[h])))
                                : static_cast<float>(static_cast<_Float16>(v * ldexpf(1.0f, qexp[h])));
      sum += rep;
    }
    P.qinit[h][c] = -8.0f * ldexpf(sum, -24);
  }
}

template <int G>
struct __align__(16) DecodeSmem {
  union alignas(16) {
    float w[kWaves][G][8][kWRow];     // per-wave weight transpose [head][block][token]
    float fold[kWaves][G][kHeadDim];  // epilogue: per-wave outputs
  } u;
  float fold_m[kWaves][G];
  float fold_l[kWaves][G];
};

static_assert((kWRow * 4) % 16 == 0, "weight rows must be 16-byte aligned");

template <int G>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a, const QPrep<G>* __restrict__ qprep) {
  __shared__ DecodeSmem<G> sm;
  const int split = blockIdx.x;
  const int b = blockIdx.y / a.Hkv;
  const int g = blockIdx.y % a.Hkv;
  const int win = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int R = gridDim.z * a.B * a.Hq;
  const int row0 = (win * a.B + b) * a.Hq + g * G;  // first output row of this group

  int ctx = a.ctx[b];
  ctx = max(0, min(ctx, a.max_ctx));
  int t0 = 0, t1 = ctx;
  if (a.window_tokens > 0) {
    t0 = win * a.window_tokens;
    t1 = min(ctx, t0 + a.window_tokens);
  }
  const int pbeg = t0 / kPage + split * a.pages_per_split;
  const int pend = min(pbeg + a.pages_per_split, (t1 + kPage - 1) / kPage);
  const int64_t out_row = static_cast<int64_t>(split) * R + row0;

  if (t1 <= t0 || pend <= pbeg) {  // nothing to attend: merge identity
    for (int i = tid; i < G * kHeadDim; i += kThreads) a.o[out_row * kHeadDim + i] = 0.0f;
    if (tid < G) {
      if (a.m) a.m[out_row + tid] = -INFINITY;
      if (a.l) a.l[out_row + tid] = 0.0f;
    }
    return;
  }

  const QPrep<G>* QP = qprep + blockIdx.y;
  float m_run[G], l_lane[G], o[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[h][d] = 0.0f;
  }
  const int cj = lane >> 3;  // block holding this lane's 4 value channels
  const int sub = lane & 7;
  const int32_t* ptrow = a.pt + static_cast<int64_t>(b) * a.max_pages;

  for (int lp = pbeg + wave; lp < pend; lp += kWaves) {
    // The query operands are re-read (scalar loads) every page.  An offset the
    // compiler cannot see through keeps it from hoisting all 512 of them out
    // of the loop, which would spill.
    int qoff = 0;
    asm volatile("" : "+s"(qoff));
    const QPrep<G>* qp = reinterpret_cast<const QPrep<G>*>(reinterpret_cast<const char*>(QP) + qoff);
    int32_t pid = ptrow[lp];
    // an out-of-range page id reads page 0 and contributes nothing
    const bool pvalid = static_cast<uint32_t>(pid) < static_cast<uint32_t>(a.num_pages);
    pid = pvalid ? pid : 0;
    const int64_t ph = static_cast<int64_t>(pid) * a.Hkv + g;
    const uint4* kt = reinterpret_cast<const uint4*>(a.k_nib + ph * (kPage * kHeadDim / 2));
    const uint4* vt = reinterpret_cast<const uint4*>(a.v_nib + ph * (kPage * kHeadDim / 2));
    uint4 kq[8], vq[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) kq[c] = kt[c * 64 + lane];
    const uint4 ks = reinterpret_cast<const uint4*>(a.k_scale + ph * (kPage * 8))[lane];
    const uint4 vs = reinterpret_cast<const uint4*>(a.v_scale + ph * (kPage * 8))[lane];
#pragma unroll
    for (int c = 0; c < 8; ++c) vq[c] = vt[c * 64 + lane];

    const int tok = lp * kPage + lane;
    const float tmask = (pvalid && tok >= t0 && tok < t1) ? 0.0f : -INFINITY;

    // keys: lane = token
    float logit[G];
#pragma unroll
    for (int h = 0; h < G; ++h) logit[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // one block's query operands (G x 16 dwords) in SGPRs at a time
      __builtin_amdgcn_sched_barrier(0);
      int qo = 0;
      asm volatile("" : "+s"(qo));
      const QPrep<G>* qb = reinterpret_cast<const QPrep<G>*>(reinterpret_cast<const char*>(qp) + qo);
      pin(kq[c]);
      const uint32_t sw = word(ks, c >> 1);
      const float sc = (c & 1) ? f16_hi(sw) : f16_lo(sw);
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = qb->qinit[h][c];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t wd = word(kq[c], k);
        const uint32_t p0 = wd & 0x000F000Fu;
        const uint32_t p1 = wd & 0x00F000F0u;
        const uint32_t w8 = wd >> 8;
        const uint32_t p2 = w8 & 0x000F000Fu;
        const uint32_t p3 = w8 & 0x00F000F0u;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h] = dot2(p0, qb->pair[h][c][k][0], acc[h]);
          acc[h] = dot2(p1, qb->pair[h][c][k][1], acc[h]);
          acc[h] = dot2(p2, qb->pair[h][c][k][2], acc[h]);
          acc[h] = dot2(p3, qb->pair[h][c][k][3], acc[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) logit[h] = fmaf(sc, acc[h], logit[h]);
    }

    // online softmax (log2 units), wave-uniform running max per head
    float alpha[G], p[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      // additive mask: written as a select, the compiler turns the whole key
      // phase into a branch on the token's validity
      const float s = fmaf(logit[h], qp->kscale[h], tmask);
      const float mn = fmaxf(m_run[h], wave_max(s));
      // mn == -inf only while no valid token has been seen: keep everything at 0
      const float ms = mn == -INFINITY ? 0.0f : mn;
      alpha[h] = __builtin_amdgcn_exp2f(m_run[h] - ms);
      p[h] = __builtin_amdgcn_exp2f(s - ms);
      l_lane[h] = fmaf(l_lane[h], alpha[h], p[h]);
      m_run[h] = mn;
    }

    // weights p * s_v per (head, block) to LDS in fp32, transposed to [head][block][token]
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t sw = word(vs, c >> 1);
      const float sv = (c & 1) ? f16_hi(sw) : f16_lo(sw);
#pragma unroll
      for (int h = 0; h < G; ++h) sm.u.w[wave][h][c][lane] = p[h] * sv;
    }
    lds_wave_sync();

    // values: lane = channels 4*lane .. 4*lane+3 (block cj)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int d = 0; d < 4; ++d) o[h][d] *= alpha[h];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      pin(vq[ct]);
      float4_t wa[G], wb[G];  // weights of tokens 8ct..8ct+3 and 8ct+4..8ct+7
#pragma unroll
      for (int h = 0; h < G; ++h) {
        wa[h] = *reinterpret_cast<const float4_t*>(&sm.u.w[wave][h][cj][ct * 8]);
        wb[h] = *reinterpret_cast<const float4_t*>(&sm.u.w[wave][h][cj][ct * 8 + 4]);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t wd = word(vq[ct], k);
        // fp16 pairs (token 8ct+2k, token 8ct+2k+1) of channels 0..3
        const half2_t v0 = __builtin_bit_cast(half2_t, wd & 0x000F000Fu);
        const half2_t v1 = __builtin_bit_cast(half2_t, wd & 0x00F000F0u);
        const uint32_t w8 = wd >> 8;
        const half2_t v2 = __builtin_bit_cast(half2_t, w8 & 0x000F000Fu);
        const half2_t v3 = __builtin_bit_cast(half2_t, w8 & 0x00F000F0u);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float w0 = k < 2 ? wa[h][2 * k] : wb[h][2 * k - 4];
          const float w1 = k < 2 ? wa[h][2 * k + 1] : wb[h][2 * k - 3];
          // fp32 weight x fp16 nibble operand, fp32 accumulate (v_fma_mix_f32)
          o[h][0] = fmaf(w1, static_cast<float>(v0.y), fmaf(w0, static_cast<float>(v0.x), o[h][0]));
          o[h][1] = fmaf(w1, static_cast<float>(v1.y), fmaf(w0, static_cast<float>(v1.x), o[h][1]));
          o[h][2] = fmaf(w1, static_cast<float>(v2.y), fmaf(w0, static_cast<float>(v2.x), o[h][2]));
          o[h][3] = fmaf(w1, static_cast<float>(v3.y), fmaf(w0, static_cast<float>(v3.x), o[h][3]));
        }
      }
    }
    // "- 8" correction: the page's summed weights of block cj
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float4_t x = *reinterpret_cast<const float4_t*>(&sm.u.w[wave][h][cj][sub * 8]);
      const float4_t y = *reinterpret_cast<const float4_t*>(&sm.u.w[wave][h][cj][sub * 8 + 4]);
      const float ws = sum8(((x.x + x.y) + (x.z + x.w)) + ((y.x + y.y) + (y.z + y.w)));
      const float c1 = ws * 4.76837158203125e-07f;  // 8 * 2^-24
      o[h][0] -= c1;
      o[h][1] -= 16.0f * c1;
      o[h][2] -= c1;
      o[h][3] -= 16.0f * c1;
    }
  }

  // ---- epilogue: fold the 4 waves, write the partial state -----------------
  float l_w[G];
#pragma unroll
  for (int h = 0; h < G; ++h) l_w[h] = wave_sum(l_lane[h]);
  __syncthreads();  // every wave is done with the weight buffers
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float4_t v;
    v.x = o[h][0] * 16777216.0f;  // 2^24
    v.y = o[h][1] * 1048576.0f;   // 2^20 (x16 slot)
    v.z = o[h][2] * 16777216.0f;
    v.w = o[h][3] * 1048576.0f;
    *reinterpret_cast<float4_t*>(&sm.u.fold[wave][h][4 * lane]) = v;
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm.fold_m[wave][h] = m_run[h];
      sm.fold_l[wave][h] = l_w[h];
    }
  }
  __syncthreads();
  for (int i = tid; i < G * kHeadDim; i += kThreads) {
    const int h = i / kHeadDim, d = i % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (sm.fold_l[w][h] > 0.0f) M = fmaxf(M, sm.fold_m[w][h]);
    float L = 0.0f, acc = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        if (sm.fold_l[w][h] > 0.0f) {
          const float e = __builtin_amdgcn_exp2f(sm.fold_m[w][h] - M);
          L = fmaf(sm.fold_l[w][h], e, L);
          acc = fmaf(sm.u.fold[w][h][d], e, acc);
        }
      }
    }
    a.o[(out_row + h) * kHeadDim + d] = L > 0.0f ? acc / L : 0.0f;
    if (d == 0) {
      if (a.m) a.m[out_row + h] = L > 0.0f ? M * kLn2 : -INFINITY;
      if (a.l) a.l[out_row + h] = L;
    }
  }
}

template <int G>
hipError_t launch_decode_g(const DecodeArgs& a, void* qprep, dim3 grid, hipStream_t s) {
  QPrep<G>* qp = static_cast<QPrep<G>*>(qprep);
  hipLaunchKernelGGL(decode_qprep_kernel<G>, dim3(a.B * a.Hkv), dim3(kThreads), 0, s, a.q, qp, a.Hq, a.Hkv,
                     a.qk_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_kernel<G>, grid, dim3(kThreads), 0, s, a, static_cast<const QPrep<G>*>(qp));
  return hipGetLastError();
}

// Workgroups of the decode kernel the current device holds at once (CUs x
// occupancy), computed once per (device, group size).
int64_t resident_workgroups(int G) {
  constexpr int kMaxDev = 64;
  static std::atomic<int64_t> cached[kMaxDev][4];
  const int gi = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
  int dev = 0, cus = 256, per = 0;
  const bool have_dev = hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDev;
  if (have_dev) {
    const int64_t c = cached[dev][gi].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  if (have_dev) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  hipError_t e = hipErrorUnknown;
  switch (G) {
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_kernel<1>, kThreads, 0); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_kernel<2>, kThreads, 0); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_kernel<4>, kThreads, 0); break;
    default: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_kernel<8>, kThreads, 0); break;
  }
  if (e != hipSuccess || per <= 0) per = 2;
  const int64_t total = static_cast<int64_t>(cus) * per;
  if (have_dev) cached[dev][gi].store(total, std::memory_order_relaxed);
  return total;
}

size_t qprep_bytes(int G, int64_t items) {
  switch (G) {
    case 1: return sizeof(QPrep<1>) * items;
    case 2: return sizeof(QPrep<2>) * items;
    case 4: return sizeof(QPrep<4>) * items;
    default: return sizeof(QPrep<8>) * items;
  }
}

}  // namespace

DecodePlan plan_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_ctx, int32_t num_windows,
                       int32_t window_tokens) {
  DecodePlan p;
  const int32_t ctx_pages = (max_ctx + kPage - 1) / kPage;
  int32_t ppw = window_tokens > 0 ? std::min(window_tokens / kPage, ctx_pages) : ctx_pages;
  ppw = std::max(ppw, 1);
  const int64_t items = static_cast<int64_t>(num_windows) * B * Hkv;
  // one full wave of workgroups: every CU holds as many as its registers allow
  const int64_t target_wgs = resident_workgroups(Hq / Hkv);
  int64_t pps = (items * ppw + target_wgs - 1) / target_wgs;
  pps = std::max<int64_t>(pps, kWaves);
  pps = std::min<int64_t>(pps, ppw);
  p.pages_per_window = ppw;
  p.pages_per_split = static_cast<int32_t>(pps);
  p.splits = static_cast<int32_t>((ppw + pps - 1) / pps);
  const int64_t R = static_cast<int64_t>(num_windows) * B * Hq;
  const size_t part = p.splits > 1 ? static_cast<size_t>(p.splits) * R * (kHeadDim + 2) * sizeof(float) : 0;
  p.qprep_offset = (part + 255) / 256 * 256;
  p.ws_bytes = p.qprep_offset + qprep_bytes(Hq / Hkv, static_cast<int64_t>(B) * Hkv);
  return p;
}

hipError_t launch_decode(const f4kv_cache& c, const uint16_t* q, const int32_t* pt, const int32_t* ctx,
                         int32_t B, int32_t Hq, int32_t max_pages, int32_t max_ctx, int32_t num_windows,
                         int32_t window_tokens, float sm_scale, float* out, float* out_m, float* out_l,
                         void* ws, const DecodePlan& plan, hipStream_t s) {
  if (B == 0) return hipSuccess;
  DecodeArgs a;
  a.k_nib = c.k_nib;
  a.k_scale = c.k_scale;
  a.v_nib = c.v_nib;
  a.v_scale = c.v_scale;
  a.q = q;
  a.pt = pt;
  a.ctx = ctx;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = c.num_kv_heads;
  a.num_pages = c.num_pages;
  a.max_pages = max_pages;
  a.max_ctx = max_ctx;
  a.window_tokens = window_tokens;
  a.pages_per_split = plan.pages_per_split;
  a.qk_scale = sm_scale * kLog2e;
  const int64_t R = static_cast<int64_t>(num_windows) * B * Hq;
  float* part_m = nullptr;
  float* part_l = nullptr;
  if (plan.splits > 1) {
    float* base = static_cast<float*>(ws);
    a.o = base;
    part_m = base + static_cast<size_t>(plan.splits) * R * kHeadDim;
    part_l = part_m + static_cast<size_t>(plan.splits) * R;
    a.m = part_m;
    a.l = part_l;
  } else {
    a.o = out;
    a.m = out_m;
    a.l = out_l;
  }
  const dim3 grid(plan.splits, B * a.Hkv, num_windows);
  const int G = Hq / a.Hkv;
  void* qprep = static_cast<char*>(ws) + plan.qprep_offset;
  hipError_t e;
  switch (G) {
    case 1: e = launch_decode_g<1>(a, qprep, grid, s); break;
    case 2: e = launch_decode_g<2>(a, qprep, grid, s); break;
    case 4: e = launch_decode_g<4>(a, qprep, grid, s); break;
    default: e = launch_decode_g<8>(a, qprep, grid, s); break;
  }
  if (e != hipSuccess || plan.splits == 1) return e;
  return launch_merge(part_m, part_l, a.o, plan.splits, static_cast<int32_t>(R), kHeadDim, out, out_m,
                      out_l, s);
}

}  // namespace f4kv
