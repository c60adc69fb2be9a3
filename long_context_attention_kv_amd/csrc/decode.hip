// paged_attn_decode_f4: split-K paged GQA decode over the F4 cache.
//
// What is computed (mistral.rs PR #2375, "Changes by area" item 2: the paged
// attention kernels read the packed F4 cells and dequantise them inline;
// FreeToken issue #568, "Proposed solution" item 2: windows folded by
// log2-sum-exp): for each (window, sequence, query head) the exact softmax
// attention of one query row over the window's cached tokens, returned as the
// partial state (m, l, o).
//
// Work split.  A small planning step (run on the device, from the context
// lengths) cuts every (window, sequence) range of pages into chunks of about
// the same length, enough of them to fill one resident wave of workgroups.  A
// workgroup of 4 waves owns one chunk of one KV head; each wave streams every
// 4th page of the chunk with its own running max / sum / output, the waves fold
// in LDS at the end, and a fold kernel combines the chunks of each output row.
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
//    value phase through LDS in fp32 and enter the products through the
//    mixed-precision FMA (fp32 weight times fp16 nibble operand): an fp16
//    weight (11 bits) would leave ~2e-3 of the output RMS on channels whose
//    values are many times the others' (outlier channels).  The "- 8" is
//    corrected once, at the end, with the summed weights of the lane's block.
// The query is pre-scaled by a power of two per head so its fp16 copy keeps
// full precision whatever its magnitude; fp32 accumulation throughout.
#include <algorithm>
#include <atomic>

#include "f4kv_internal.h"

namespace f4kv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kWRow = 68;  // fp32 weights per (head, block) row: 64 tokens + 16 B pad
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.0f;  // log2 units a logit may exceed the running max by

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
  const int4* items;       // work items (window * B + sequence, first page, end page, first item of the range)
  const int32_t* n_items;  // number of valid items
  const int32_t* count;    // [W * B] items of each (window, sequence)
  float* o;                // partial outputs [item][Hr][D]
  float* m;                // [item][Hr], log2 units
  float* l;                // [item][Hr]
  float* out;              // [W * B][Hr][D]
  float* out_m;            // [W * B][Hr] or null
  float* out_l;            // [W * B][Hr] or null
  int32_t B, Hq, Hkv, num_pages, max_pages, max_ctx;
  // query rows: R per sequence (row r at position ctx - R + r), Hr = R * Hq
  // output rows per range (row r, head h at r * Hq + h); this launch computes
  // rows r0 .. r0 + G / Gq - 1 (Gq = Hq / Hkv query heads per KV head)
  int32_t R, r0, Gq, Hr;
  int32_t window_tokens;
  float qk_scale;  // sm_scale * log2(e)
};

// The work list: every (window, sequence) range of pages is cut into chunks of
// about the same number of pages, sized from the actual context lengths (read
// on the device) so that all chunks of all KV heads fill one resident wave of
// workgroups.  A ragged batch is thus balanced by pages, not by sequences.
struct PlanArgs {
  const int32_t* ctx;
  int4* items;
  int32_t* first;    // [W * B] first item of each (window, sequence)
  int32_t* count;    // [W * B] its number of items
  int32_t* n_items;
  float* out;        // rows of empty ranges are written here
  float* out_m;
  float* out_l;
  int32_t B, W, Hr, Hkv, window_tokens, max_ctx, per_head_target;  // Hr: output rows per range
};

__device__ __forceinline__ void window_pages(const PlanArgs& p, int wb, int& p0, int& p1) {
  const int b = wb % p.B, w = wb / p.B;
  const int ctx = max(0, min(p.ctx[b], p.max_ctx));
  int t0 = 0, t1 = ctx;
  if (p.window_tokens > 0) {
    t0 = w * p.window_tokens;
    t1 = min(ctx, t0 + p.window_tokens);
  }
  p0 = t0 / kPage;
  p1 = t1 > t0 ? (t1 + kPage - 1) / kPage : p0;
}

__device__ int64_t block_sum(int64_t v, int64_t* s64) {
  const int tid = threadIdx.x;
  __syncthreads();
  s64[tid] = v;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) s64[tid] += s64[tid + w];
    __syncthreads();
  }
  return s64[0];
}

// Number of chunks when every range is cut into pieces of at most pps pages.
__device__ int64_t count_chunks(const PlanArgs& p, int pps, int64_t* s64) {
  int64_t c = 0;
  for (int wb = threadIdx.x; wb < p.W * p.B; wb += kThreads) {
    int p0, p1;
    window_pages(p, wb, p0, p1);
    c += (p1 - p0 + pps - 1) / pps;
  }
  return block_sum(c, s64);
}

// Run by one workgroup of kThreads threads.  The chunk length is the smallest
// one (at least kWaves pages) whose chunk count fits the per-head target; the
// pages of a range are then shared evenly among its chunks.  Ranges with no
// tokens get no item; their output rows are written here (m = -inf, l = 0,
// o = 0).
__device__ void build_work_list(const PlanArgs& p) {
  __shared__ int64_t s64[kThreads];
  __shared__ int32_t s_end[kThreads];  // inclusive scan of the chunk counts of a batch of ranges
  __shared__ int32_t s_p0[kThreads], s_len[kThreads];
  const int tid = threadIdx.x;
  const int n = p.W * p.B;
  int64_t total = 0;
  for (int wb = tid; wb < n; wb += kThreads) {
    int p0, p1;
    window_pages(p, wb, p0, p1);
    total += p1 - p0;
  }
  total = block_sum(total, s64);
  const int64_t target = p.per_head_target;
  int64_t lo = max<int64_t>(kWaves, (total + target - 1) / target);
  // with chunks of hi pages the rounding adds at most one chunk per range
  int64_t hi = target > n ? max<int64_t>(lo, (total + target - n - 1) / (target - n)) : lo;
  while (lo < hi) {  // smallest length in [lo, hi] whose count fits
    const int64_t mid = (lo + hi) / 2;
    if (count_chunks(p, static_cast<int>(mid), s64) <= target)
      hi = mid;
    else
      lo = mid + 1;
  }
  const int pps = static_cast<int>(lo);
  int base = 0;
  for (int t0 = 0; t0 < n; t0 += kThreads) {
    const int wb = t0 + tid;
    int p0 = 0, p1 = 0, chunks = 0;
    if (wb < n) {
      window_pages(p, wb, p0, p1);
      chunks = (p1 - p0 + pps - 1) / pps;
    }
    __syncthreads();
    s_end[tid] = chunks;
    s_p0[tid] = p0;
    s_len[tid] = p1 - p0;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int v = tid >= off ? s_end[tid - off] : 0;
      __syncthreads();
      s_end[tid] += v;
      __syncthreads();
    }
    const int batch = s_end[kThreads - 1];
    if (wb < n) {
      p.first[wb] = base + s_end[tid] - chunks;
      p.count[wb] = chunks;
    }
    if (__syncthreads_count(wb < n && chunks == 0)) {  // identity rows of empty ranges
      for (int r = 0; r < kThreads && t0 + r < n; ++r) {
        if (s_len[r] > 0) continue;
        const int64_t r0 = static_cast<int64_t>(t0 + r) * p.Hr;
        for (int i = tid; i < p.Hr * kHeadDim; i += kThreads) p.out[r0 * kHeadDim + i] = 0.0f;
        for (int i = tid; i < p.Hr; i += kThreads) {
          if (p.out_m) p.out_m[r0 + i] = -INFINITY;
          if (p.out_l) p.out_l[r0 + i] = 0.0f;
        }
      }
    }
    // item j of the batch belongs to the first range whose running count exceeds j
    for (int j = tid; j < batch; j += kThreads) {
      int r = 0;
      for (int step = kThreads / 2; step > 0; step >>= 1)
        if (s_end[r + step - 1] <= j) r += step;
      const int c_cnt = s_end[r] - (r ? s_end[r - 1] : 0);
      const int c = j - (s_end[r] - c_cnt);
      const int len = s_len[r], q = len / c_cnt, rem = len % c_cnt;
      const int beg = s_p0[r] + c * q + min(c, rem);
      const int end = beg + q + (c < rem ? 1 : 0);
      p.items[base + j] = make_int4(t0 + r, beg, end, base + j - c);
    }
    base += batch;
    __syncthreads();
  }
  if (tid == 0) *p.n_items = base;
}

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

// Raw buffer resource over `bytes` bytes at a wave-uniform address (gfx9
// descriptor: 32-bit data, no swizzle); loads beyond `bytes` return 0 without
// touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 16 bytes at lane_offset + uniform_offset (the latter in a scalar register).
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int lane_offset, int uniform_offset = 0) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, lane_offset, uniform_offset, 0));
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
// Workgroups 0 .. B*Hkv-1 prepare the query operands of one (sequence, KV
// head) each; the last workgroup builds the work list.
template <int G>
__global__ __launch_bounds__(kThreads) void decode_qprep_kernel(const uint16_t* __restrict__ q,
                                                               QPrep<G>* __restrict__ out, int32_t Hq,
                                                               int32_t Hkv, float qk_scale, PlanArgs plan,
                                                               int32_t R, int32_t r0, int32_t Gq) {
  if (blockIdx.x == gridDim.x - 1) {
    build_work_list(plan);
    return;
  }
  __shared__ float qf[G][kHeadDim];
  __shared__ int32_t qexp[G];
  const int b = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  QPrep<G>& P = out[blockIdx.x];
  // row h of the group: query row r0 + h / Gq (clamped: rows past R are computed, never written), head g Gq + h % Gq
  for (int i = tid; i < G * kHeadDim; i += kThreads) {
    const int h = i / kHeadDim, r = min(r0 + h / Gq, R - 1);
    const int64_t row = (static_cast<int64_t>(b) * R + r) * Hq + g * Gq + h % Gq;
    qf[h][i % kHeadDim] = bf16_to_f32(q[row * kHeadDim + i % kHeadDim]);
  }
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

// Combines the per-wave states in LDS (max in log2 units, sum, normalised
// output) into the group's rows of dst: row h of the group is output row
// rowbase + (r0 + h / Gq) * Hq + g * Gq + h % Gq (rows past R are dropped):
// the output (max in natural log) when final, else a partial state (max in
// log2 units).
template <int G>
__device__ __forceinline__ void fold_waves(const DecodeSmem<G>& sm, float* dst, int64_t rowbase, const DecodeArgs& a,
                                           int g, bool final) {
  for (int i = threadIdx.x; i < G * kHeadDim; i += kThreads) {
    const int h = i / kHeadDim, d = i % kHeadDim;
    const int r = a.r0 + h / a.Gq;
    if (r >= a.R) continue;
    const int64_t row = rowbase + static_cast<int64_t>(r) * a.Hq + g * a.Gq + h % a.Gq;
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
    dst[row * kHeadDim + d] = L > 0.0f ? acc / L : 0.0f;
    if (d == 0) {
      if (final) {
        if (a.out_m) a.out_m[row] = L > 0.0f ? M * kLn2 : -INFINITY;
        if (a.out_l) a.out_l[row] = L;
      } else {
        a.m[row] = L > 0.0f ? M : -INFINITY;
        a.l[row] = L;
      }
    }
  }
}

static_assert((kWRow * 4) % 16 == 0, "weight rows must be 16-byte aligned");

// VT: V scales are one per token and head (v_scale [P][H][64]) instead of one
// per 32 values; the weight of a token is then the same for all blocks, so a
// single row of weights per head goes through LDS.
template <int G, bool VT>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a, const QPrep<G>* __restrict__ qprep) {
  __shared__ DecodeSmem<G> sm;
  const int item = blockIdx.x;
  const int g = blockIdx.y;
  if (item >= *a.n_items) return;
  const int4 it_v = a.items[item];
  // the work item is wave-uniform: keep it (and all that derives from it) in SGPRs
  const int4 it = make_int4(__builtin_amdgcn_readfirstlane(it_v.x), __builtin_amdgcn_readfirstlane(it_v.y),
                            __builtin_amdgcn_readfirstlane(it_v.z), __builtin_amdgcn_readfirstlane(it_v.w));
  const int b = __builtin_amdgcn_readfirstlane(it.x % a.B);
  const int win = __builtin_amdgcn_readfirstlane(it.x / a.B);
  const int pbeg = it.y, pend = it.z;
  const int nchunks = a.count[it.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so page ids load as scalars

  int ctx = a.ctx[b];
  ctx = max(0, min(ctx, a.max_ctx));
  int t0 = 0, t1 = ctx;
  if (a.window_tokens > 0) {
    t0 = win * a.window_tokens;
    t1 = min(ctx, t0 + a.window_tokens);
  }

  // last token + 1 that each row of the group sees: row r sits at ctx - R + r
  int lim[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    lim[h] = __builtin_amdgcn_readfirstlane(min(t1, ctx - (a.R - 1 - (a.r0 + h / a.Gq))));

  const QPrep<G>* QP = qprep + __builtin_amdgcn_readfirstlane(b * a.Hkv + g);
  float m_run[G], s_max[G], l_lane[G], o[G][4];
  float wpart[G];  // this lane's share (8 tokens of each page) of the summed weights of block cj
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    s_max[h] = -INFINITY;
    l_lane[h] = 0.0f;
    wpart[h] = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[h][d] = 0.0f;
  }
  const int cj = lane >> 3;  // block holding this lane's 4 value channels
  const int sub = lane & 7;
  const int32_t* ptrow = a.pt + static_cast<int64_t>(b) * a.max_pages;
  const int lane16 = lane * 16;

  for (int lp = pbeg + wave; lp < pend; lp += kWaves) {
    // The query operands are re-read (scalar loads) every page.  An offset the
    // compiler cannot see through keeps it from hoisting all 512 of them out
    // of the loop, which would spill.
    int qoff = 0;
    asm volatile("" : "+s"(qoff));
    const QPrep<G>* qp = reinterpret_cast<const QPrep<G>*>(reinterpret_cast<const char*>(QP) + qoff);
    // Tiles of this page through buffer resources with a scalar base: the lane
    // offsets are constants, so no per-page address arithmetic runs on the VALU.
    // An out-of-range page id gets empty resources (loads return 0, no traffic)
    // and a mask that drops its tokens.
    const int32_t pid = ptrow[lp];
    const bool pvalid = static_cast<uint32_t>(pid) < static_cast<uint32_t>(a.num_pages);
    const int64_t ph = static_cast<int64_t>(pvalid ? pid : 0) * a.Hkv + g;
    const int tile_bytes = pvalid ? kPage * kHeadDim / 2 : 0;
    const int scale_bytes = pvalid ? kPage * 8 * 2 : 0;
    const auto rk = tile_rsrc(a.k_nib + ph * (kPage * kHeadDim / 2), tile_bytes);
    const auto rv = tile_rsrc(a.v_nib + ph * (kPage * kHeadDim / 2), tile_bytes);
    uint4 kq[8], vq[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) kq[c] = load16(rk, lane16, c * 1024);
    __builtin_amdgcn_s_setprio(0);
    const uint4 ks = load16(tile_rsrc(a.k_scale + ph * (kPage * 8), scale_bytes), lane16);
    uint4 vs = make_uint4(0, 0, 0, 0);
    uint32_t vs1 = 0;  // this token's V scale (VT)
    if (VT)
      vs1 = __builtin_amdgcn_raw_buffer_load_b16(tile_rsrc(a.v_scale + ph * kPage, pvalid ? kPage * 2 : 0),
                                                 lane * 2, 0, 0);
    else
      vs = load16(tile_rsrc(a.v_scale + ph * (kPage * 8), scale_bytes), lane16);

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

    // the values are requested only now, so they do not hold registers through
    // the key phase (other waves cover their latency)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 8; ++c) vq[c] = load16(rv, lane16, c * 1024);

    // Online softmax in log2 units with a lazily raised running max: m_run
    // moves (and the state is rescaled) only when some logit of the page
    // exceeds it by more than kSlack, so weights stay below 2^kSlack and
    // most pages skip the wave-wide max and the rescale.  The exact maximum is
    // tracked per lane and restored at the end.
    float p[G], s[G];
    bool raise = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      // additive mask: written as a select, the compiler turns the whole key
      // phase into a branch on the token's validity
      s[h] = fmaf(logit[h], qp->kscale[h], tok < lim[h] ? tmask : -INFINITY);
      s_max[h] = fmaxf(s_max[h], s[h]);
      raise |= s[h] > m_run[h] + kSlack;
    }
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m_run[h], wave_max(s[h]));
        // mn == -inf only while no valid token has been seen: nothing to rescale
        const float alpha = m_run[h] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[h] - mn);
        l_lane[h] *= alpha;
        wpart[h] *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d) o[h][d] *= alpha;
        m_run[h] = mn;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      p[h] = __builtin_amdgcn_exp2f(s[h] - (m_run[h] == -INFINITY ? 0.0f : m_run[h]));
      l_lane[h] += p[h];
    }

    // weights p * s_v per (head, block) to LDS in fp32, transposed to
    // [head][block][token] (VT: one block row per head)
    if (VT) {
      const float sv = f16_lo(vs1);
#pragma unroll
      for (int h = 0; h < G; ++h) sm.u.w[wave][h][0][lane] = p[h] * sv;
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t sw = word(vs, c >> 1);
        const float sv = (c & 1) ? f16_hi(sw) : f16_lo(sw);
#pragma unroll
        for (int h = 0; h < G; ++h) sm.u.w[wave][h][c][lane] = p[h] * sv;
      }
    }
    lds_wave_sync();
    const int wrow = VT ? 0 : cj;  // weight row of this lane's value block

    // values: lane = channels 4*lane .. 4*lane+3 (block cj); this wave's VALU
    // stream goes first while it holds its operands
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      if ((ct & 1) == 0) __builtin_amdgcn_sched_barrier(0);  // two token groups' weights in flight
      pin(vq[ct]);
      float4_t wa[G], wb[G];  // weights of tokens 8ct..8ct+3 and 8ct+4..8ct+7
#pragma unroll
      for (int h = 0; h < G; ++h) {
        wa[h] = *reinterpret_cast<const float4_t*>(&sm.u.w[wave][h][wrow][ct * 8]);
        wb[h] = *reinterpret_cast<const float4_t*>(&sm.u.w[wave][h][wrow][ct * 8 + 4]);
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
    // "- 8" correction, part 1: this lane's 8 tokens of the page's weights of
    // block cj (the 8 lanes of the block cover its 64 tokens); the sum over the
    // lanes and the correction itself wait for the epilogue
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float4_t x = *reinterpret_cast<const float4_t*>(&sm.u.w[wave][h][wrow][sub * 8]);
      const float4_t y = *reinterpret_cast<const float4_t*>(&sm.u.w[wave][h][wrow][sub * 8 + 4]);
      wpart[h] += ((x.x + x.y) + (x.z + x.w)) + ((y.x + y.y) + (y.z + y.w));
    }
  }

  // "- 8" correction, part 2: the summed weights of block cj over every page of
  // the wave, times 8 (in the units of the nibble operands, 2^-24 and 16 x 2^-24)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float c1 = sum8(wpart[h]) * 4.76837158203125e-07f;  // 8 * 2^-24
    o[h][0] -= c1;
    o[h][1] -= 16.0f * c1;
    o[h][2] -= c1;
    o[h][3] -= 16.0f * c1;
  }

  // ---- epilogue: restore the exact maximum, fold the 4 waves ---------------
  __builtin_amdgcn_s_setprio(0);
  float l_w[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mx = wave_max(s_max[h]);  // <= m_run + kSlack
    if (mx != -INFINITY) {
      const float f = __builtin_amdgcn_exp2f(m_run[h] - mx);
      l_lane[h] *= f;
#pragma unroll
      for (int d = 0; d < 4; ++d) o[h][d] *= f;
      m_run[h] = mx;
    }
    l_w[h] = wave_sum(l_lane[h]);
  }
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
  // A range of a single item writes its output rows directly; otherwise the
  // item writes its partial state for the fold kernel.
  const bool single = nchunks == 1;
  fold_waves<G>(sm, single ? a.out : a.o, static_cast<int64_t>(single ? it.x : item) * a.Hr, a, g, single);
}

constexpr int kFoldWaves = 16;

// Folds the partial states of each output row (window, sequence, query row,
// query head) whose range has two or more items: items first[wb] .. first[wb]
// + count[wb] - 1, maxima in log2 units.  Workgroup x folds row (x / (Rp Hq))
// * Hr + (r0 + x % (Rp Hq) / Hq) * Hq + x % Hq: the rows r0 .. r0 + Rp - 1 of
// this launch.  Wave w takes every 16th item with a running max (lane = 4
// channels); the 16 wave states meet in LDS.
__global__ __launch_bounds__(64 * kFoldWaves) void decode_fold_kernel(const float* __restrict__ po,
                                                                     const float* __restrict__ pm,
                                                                     const float* __restrict__ pl,
                                                                     const int32_t* __restrict__ first,
                                                                     const int32_t* __restrict__ count,
                                                                     int32_t Hr, int32_t r0, int32_t Rp,
                                                                     int32_t Hq, float* out, float* out_m,
                                                                     float* out_l) {
  const int x = blockIdx.x;
  const int wb = x / (Rp * Hq);
  const int rr = (r0 + (x % (Rp * Hq)) / Hq) * Hq + x % Hq;  // row within the range
  const int64_t r = static_cast<int64_t>(wb) * Hr + rr;       // output row
  const int n = count[wb];
  if (n < 2) return;  // written by the decode kernel or the planning step
  const int c0 = first[wb];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __shared__ float4_t s_acc[kFoldWaves][64];
  __shared__ float s_m[kFoldWaves], s_l[kFoldWaves];
  float Mr = -INFINITY, Lr = 0.0f;
  float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int c = wave; c < n; c += kFoldWaves) {
    const int64_t i = static_cast<int64_t>(c0 + c) * Hr + rr;
    const float mi = pm[i], li = pl[i];
    const float4_t oi = reinterpret_cast<const float4_t*>(po + i * kHeadDim)[lane];
    const float Mn = li > 0.0f ? fmaxf(Mr, mi) : Mr;
    const float sc = Mr == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(Mr - Mn);
    const float wi = li > 0.0f ? li * __builtin_amdgcn_exp2f(mi - Mn) : 0.0f;
    acc = acc * sc + oi * wi;
    Lr = Lr * sc + wi;
    Mr = Mn;
  }
  s_acc[wave][lane] = acc;
  if (lane == 0) {
    s_m[wave] = Mr;
    s_l[wave] = Lr;
  }
  __syncthreads();
  if (wave != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kFoldWaves; ++w)
    if (s_l[w] > 0.0f) M = fmaxf(M, s_m[w]);
  float L = 0.0f;
  float4_t at = float4_t{0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kFoldWaves; ++w) {
      if (s_l[w] > 0.0f) {
        const float e = __builtin_amdgcn_exp2f(s_m[w] - M);
        L = fmaf(s_l[w], e, L);
        at += s_acc[w][lane] * e;
      }
    }
  }
  reinterpret_cast<float4_t*>(out + static_cast<int64_t>(r) * kHeadDim)[lane] = L > 0.0f ? at / L : at * 0.0f;
  if (lane == 0) {
    if (out_m) out_m[r] = L > 0.0f ? M * kLn2 : -INFINITY;
    if (out_l) out_l[r] = L;
  }
}

template <int G, bool VT>
hipError_t launch_decode_g(const DecodeArgs& a, void* qprep, const PlanArgs& plan, int max_items,
                           hipStream_t s) {
  QPrep<G>* qp = static_cast<QPrep<G>*>(qprep);
  hipLaunchKernelGGL(decode_qprep_kernel<G>, dim3(a.B * a.Hkv + 1), dim3(kThreads), 0, s, a.q, qp, a.Hq, a.Hkv,
                     a.qk_scale, plan, a.R, a.r0, a.Gq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  timing_begin(F4KV_KERNEL_DECODE, s);
  hipLaunchKernelGGL((decode_kernel<G, VT>), dim3(max_items, a.Hkv), dim3(kThreads), 0, s, a,
                     static_cast<const QPrep<G>*>(qp));
  e = hipGetLastError();
  timing_end(F4KV_KERNEL_DECODE, s);
  return e;
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
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_kernel<1, false>, kThreads, 0); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_kernel<2, false>, kThreads, 0); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_kernel<4, false>, kThreads, 0); break;
    default: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_kernel<8, false>, kThreads, 0); break;
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

// Rows per launch: the kernel's row group is G = Gq * rows (query heads per
// KV head times query rows), at most 8; more rows take several launches over
// the same pages.
int rows_per_launch(int32_t R, int32_t Gq) { return std::max(1, std::min<int32_t>(R, 8 / Gq)); }

int group_size(int32_t R, int32_t Gq) {
  const int g = rows_per_launch(R, Gq) * Gq;
  return g <= 1 ? 1 : g <= 2 ? 2 : g <= 4 ? 4 : 8;
}

}  // namespace

DecodePlan plan_decode(int32_t B, int32_t R, int32_t Hq, int32_t Hkv, int32_t max_ctx, int32_t num_windows,
                       int32_t window_tokens) {
  (void)max_ctx;
  (void)window_tokens;
  DecodePlan p;
  const int G = group_size(R, Hq / Hkv);
  // all chunks of all KV heads fill one resident wave of workgroups
  const int64_t target_wgs = resident_workgroups(G);
  p.per_head_target = static_cast<int32_t>(std::max<int64_t>(1, target_wgs / Hkv));
  const int64_t wb = static_cast<int64_t>(num_windows) * B;
  p.max_items = static_cast<int32_t>(wb + p.per_head_target + 1);
  const int64_t Hr = static_cast<int64_t>(R) * Hq;
  auto align = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  p.part_o_offset = off;
  off = align(off + static_cast<size_t>(p.max_items) * Hr * kHeadDim * sizeof(float));
  p.part_ml_offset = off;
  off = align(off + static_cast<size_t>(p.max_items) * Hr * 2 * sizeof(float));
  p.items_offset = off;
  off = align(off + static_cast<size_t>(p.max_items) * sizeof(int4));
  p.count_offset = off;  // first [W * B], count [W * B], n_items
  off = align(off + static_cast<size_t>(wb) * 2 * sizeof(int32_t) + sizeof(int32_t));
  p.qprep_offset = off;
  off = align(off + qprep_bytes(G, static_cast<int64_t>(B) * Hkv));
  p.ws_bytes = off;
  return p;
}

hipError_t launch_decode(const f4kv_cache& c, const uint16_t* q, const int32_t* pt, const int32_t* ctx,
                         int32_t B, int32_t R, int32_t Hq, int32_t max_pages, int32_t max_ctx, int32_t num_windows,
                         int32_t window_tokens, float sm_scale, float* out, float* out_m, float* out_l,
                         void* ws, const DecodePlan& plan, hipStream_t s) {
  if (B == 0) return hipSuccess;
  char* base = static_cast<char*>(ws);
  const int64_t wb = static_cast<int64_t>(num_windows) * B;
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
  a.qk_scale = sm_scale * kLog2e;
  a.R = R;
  a.Gq = Hq / a.Hkv;
  a.Hr = R * Hq;
  a.o = reinterpret_cast<float*>(base + plan.part_o_offset);
  a.m = reinterpret_cast<float*>(base + plan.part_ml_offset);
  a.l = a.m + static_cast<size_t>(plan.max_items) * a.Hr;
  int4* items = reinterpret_cast<int4*>(base + plan.items_offset);
  int32_t* first = reinterpret_cast<int32_t*>(base + plan.count_offset);
  int32_t* count = first + wb;
  int32_t* n_items = count + wb;
  a.items = items;
  a.n_items = n_items;
  a.count = count;
  a.out = out;
  a.out_m = out_m;
  a.out_l = out_l;
  PlanArgs pa;
  pa.ctx = ctx;
  pa.items = items;
  pa.first = first;
  pa.count = count;
  pa.n_items = n_items;
  pa.out = out;
  pa.out_m = out_m;
  pa.out_l = out_l;
  pa.B = B;
  pa.W = num_windows;
  pa.Hr = a.Hr;
  pa.Hkv = a.Hkv;
  pa.window_tokens = window_tokens;
  pa.max_ctx = max_ctx;
  pa.per_head_target = plan.per_head_target;
  void* qprep = base + plan.qprep_offset;
  const int G = group_size(R, a.Gq);
  const int Rp = rows_per_launch(R, a.Gq);
  const bool vt = c.v_scale_per_token != 0;
  for (int r0 = 0; r0 < R; r0 += Rp) {
    a.r0 = r0;
    hipError_t e;
    switch (G) {
      case 1: e = vt ? launch_decode_g<1, true>(a, qprep, pa, plan.max_items, s)
                     : launch_decode_g<1, false>(a, qprep, pa, plan.max_items, s); break;
      case 2: e = vt ? launch_decode_g<2, true>(a, qprep, pa, plan.max_items, s)
                     : launch_decode_g<2, false>(a, qprep, pa, plan.max_items, s); break;
      case 4: e = vt ? launch_decode_g<4, true>(a, qprep, pa, plan.max_items, s)
                     : launch_decode_g<4, false>(a, qprep, pa, plan.max_items, s); break;
      default: e = vt ? launch_decode_g<8, true>(a, qprep, pa, plan.max_items, s)
                      : launch_decode_g<8, false>(a, qprep, pa, plan.max_items, s); break;
    }
    if (e != hipSuccess) return e;
    const int rows = std::min(Rp, R - r0);
    hipLaunchKernelGGL(decode_fold_kernel, dim3(static_cast<unsigned>(wb * rows * Hq)), dim3(64 * kFoldWaves), 0, s,
                       a.o, a.m, a.l, first, count, a.Hr, r0, rows, Hq, out, out_m, out_l);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace f4kv
