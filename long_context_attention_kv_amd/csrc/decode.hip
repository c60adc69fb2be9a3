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
//    block-major K tile); the G logits are formed on the matrix cores with
//    the 4 x 4 x 4 fp16 product in 16 blocks, whose lane layout is exactly
//    lane = token (4 tokens per block, A = 4 query heads x 4 channels, read
//    from LDS).  A nibble n becomes an exact fp16 operand with one AND:
//    0x000F000F picks two nibbles into the mantissas of an fp16 pair, i.e. the
//    subnormals n * 2^-24; 0x00F000F0 picks the next two as 16 n * 2^-24 (the
//    matching query pair is pre-divided by 16).  The "- 8" of every code is
//    one term per (head, block), -8 2^-24 times the sum of the block's query
//    operands, prepared with the query and used as the accumulator's start.
//    The block scale is applied once per block.  This takes the 512 dot
//    products per page off the vector ALUs, which otherwise bound the kernel
//    below the memory rate.
//  * values: lane = 4 consecutive channels, on the matrix cores as well.  The
//    V tile stores 8 tokens x 4 channels per 16-byte unit, two tokens per
//    dword, so the same masks and add yield fp16 pairs (n - 8) * 2^-24 (x16
//    for two of the channels) over two tokens: two dwords give one channel
//    over 4 tokens, a column of the 4 x 4 x 4 product.  The weights
//    w = p_t * s_t (softmax weight times the token's block scale) travel from
//    the key phase to the value phase through LDS in fp32 and are turned into
//    fp16 pairs hi + lo per (page, head, block), in units of the block's
//    largest weight (about 21 bits each; a single fp16 weight, 11 bits, would
//    leave ~2e-3 of the output RMS on channels whose values are many times
//    the others').
//    These operands are centred (n - 8, one packed fp16 add of -8 2^-24 per
//    pair) because the 4 x 4 x 4 product sums with a relative error of ~2^-19
//    (measured), which the cancellation of sum w n against 8 sum w would
//    multiply on channels whose outputs are near zero (the weights w are all
//    positive).  The keys need no such care: the query's signs already make
//    sum q n and 8 sum q of the same order as their difference, and the
//    measured errors equal those of centred keys.
// The query is pre-scaled by a power of two per head so its fp16 copy keeps
// full precision whatever its magnitude; fp32 accumulation throughout.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "f4kv_device.h"

namespace f4kv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kWRow = 68;  // fp32 weights per (head, block) row: 64 tokens + 16 B pad
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.0f;  // log2 units a logit may exceed the running max by
constexpr int kNumBlocks = kHeadDim / kBlock;  // scale blocks per head row

// Query operands of one (sequence, KV head), prepared once per call: the
// decode kernel copies the pairs to LDS (each lane reads its head's row as
// matrix-core operands) and reads the logit scales with scalar loads.
template <int G>
struct __align__(64) QPrep {
  uint32_t pair[G][8][4][4];  // fp16 pairs [head][block][dword][pair], scaled by 2^e_h
  float kscale[G];            // 2^(24 - e_h) * sm_scale * log2(e)
  float k8[8][G];             // per block and head: -8 2^-24 times the sum of the query operands
};

// The new token of each sequence for a decode step (paged_attn_decode_step_f4):
// cos / sin rows [B][rd/2] at its position, q not yet rotated, k_new / v_new
// fp32 [B][Hkv][D] (k not yet rotated), slots [B].  cos == null: no step.
struct StepArgs {
  const float* cos;
  const float* sin;
  int32_t rd;
  const float* k_new;
  const float* v_new;
  const int32_t* slots;
  uint8_t* k_nib;
  uint16_t* k_scale;
  uint8_t* v_nib;
  uint16_t* v_scale;
  int32_t num_pages, v_per_token;
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

// The same work list, built by one wave when there are at most 64 (window,
// sequence) ranges (lane r owns range r): reductions and the prefix sum run
// on the wave's shuffles, with no workgroup barrier.
__device__ int64_t wave_sum64(int64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ void build_work_list_wave(const PlanArgs& p) {
  __shared__ int32_t s_end[64], s_p0[64], s_len[64];
  const int lane = threadIdx.x;
  const int n = p.W * p.B;
  int p0 = 0, p1 = 0;
  if (lane < n) window_pages(p, lane, p0, p1);
  const int len = p1 - p0;
  const int64_t total = wave_sum64(len);
  const int64_t target = p.per_head_target;
  int64_t lo = max<int64_t>(kWaves, (total + target - 1) / target);
  int64_t hi = target > n ? max<int64_t>(lo, (total + target - n - 1) / (target - n)) : lo;
  while (lo < hi) {  // smallest length in [lo, hi] whose chunk count fits
    const int64_t mid = (lo + hi) / 2;
    if (wave_sum64(lane < n ? (len + mid - 1) / mid : 0) <= target)
      hi = mid;
    else
      lo = mid + 1;
  }
  const int pps = static_cast<int>(lo);
  const int chunks = lane < n ? (len + pps - 1) / pps : 0;
  int incl = chunks;  // inclusive prefix sum over the lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  s_end[lane] = incl;
  s_p0[lane] = p0;
  s_len[lane] = len;
  if (lane < n) {
    p.first[lane] = incl - chunks;
    p.count[lane] = chunks;
  }
  const int items = __shfl(incl, 63, 64);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // identity rows of the empty ranges
  uint64_t empty = __ballot(lane < n && len == 0);
  while (empty) {
    const int r = __builtin_ctzll(empty);
    empty &= empty - 1;
    const int64_t r0 = static_cast<int64_t>(r) * p.Hr;
    for (int i = lane; i < p.Hr * kHeadDim; i += 64) p.out[r0 * kHeadDim + i] = 0.0f;
    for (int i = lane; i < p.Hr; i += 64) {
      if (p.out_m) p.out_m[r0 + i] = -INFINITY;
      if (p.out_l) p.out_l[r0 + i] = 0.0f;
    }
  }
  // item j belongs to the first range whose running count exceeds j
  for (int j = lane; j < items; j += 64) {
    int r = 0;
#pragma unroll
    for (int step = 32; step > 0; step >>= 1)
      if (s_end[r + step - 1] <= j) r += step;
    const int c_cnt = s_end[r] - (r ? s_end[r - 1] : 0);
    const int c = j - (s_end[r] - c_cnt);
    const int ln = s_len[r], q = ln / c_cnt, rem = ln % c_cnt;
    const int beg = s_p0[r] + c * q + min(c, rem);
    const int end = beg + q + (c < rem ? 1 : 0);
    p.items[j] = make_int4(r, beg, end, j - c);
  }
  if (lane == 0) *p.n_items = items;
}

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __fp16 pk16_t __attribute__((ext_vector_type(2)));  // v_cvt_pkrtz_f16_f32's result
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// v_mfma_f32_4x4x4_16b_f16: 16 independent 4 x 4 x 4 products.  Lane 4 b + i
// gives row i of block b's A (4 fp16 in a0, a1), lane 4 b + j column j of its
// B (b0, b1); lane 4 b + j receives D[i][j] in element i.  With A = 4 query
// heads (the same in every block) and B = the masked nibbles of token 4 b + j
// (= the lane), element h of the result is head h's partial logit of the
// lane's own token.  fp16 subnormal operands (the masked nibbles) are exact.
__device__ __forceinline__ float4_t mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, float4_t c) {
  u32x2_t a, b;
  a.x = a0;
  a.y = a1;
  b.x = b0;
  b.y = b1;
  return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, a), __builtin_bit_cast(half4_t, b), c, 0, 0,
                                            0);
}

// x - bias on two fp16 lanes (v_pk_add_f16 with the negated bias).
constexpr uint32_t kM8 = 0x80088008u;    // -8 2^-24 in both halves
constexpr uint32_t kM128 = 0x80808080u;  // -128 2^-24 (the x16 slots)
__device__ __forceinline__ uint32_t centre(uint32_t x, uint32_t neg_bias) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, x) + __builtin_bit_cast(half2_t, neg_bias));
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

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kCtrl, 0xF, 0xF, false));
}

// Max of non-negative fp32 values over each group of 8 consecutive lanes,
// returned in all 8.  Non-negative floats order as their bit patterns, so the
// max runs on integers (no NaN quieting around each step).
__device__ __forceinline__ float max8_nonneg(float4_t x, float4_t y) {
  const uint32_t a = max(max(__float_as_uint(x.x), __float_as_uint(x.y)), max(__float_as_uint(x.z), __float_as_uint(x.w)));
  const uint32_t b = max(max(__float_as_uint(y.x), __float_as_uint(y.y)), max(__float_as_uint(y.z), __float_as_uint(y.w)));
  uint32_t m = max(a, b);
  m = max(m, dpp_u<kDppQuadXor1>(m));
  m = max(m, dpp_u<kDppQuadXor2>(m));
  m = max(m, dpp_u<kDppHalfMirror>(m));
  return __uint_as_float(m);
}

// Floats as int32 keys of the same order (negative values have their
// magnitude bits flipped), so that maxima run on integer DPP max without the
// float max's operand canonicalisation.
__device__ __forceinline__ int32_t order_key(float x) {
  const int32_t b = __float_as_int(x);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}

__device__ __forceinline__ float key_value(int32_t k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }

// Largest key of the wave (uniform).
__device__ __forceinline__ int32_t wave_max_key(int32_t k) {
  k = max(k, static_cast<int32_t>(dpp_u<kDppQuadXor1>(static_cast<uint32_t>(k))));
  k = max(k, static_cast<int32_t>(dpp_u<kDppQuadXor2>(static_cast<uint32_t>(k))));
  k = max(k, static_cast<int32_t>(dpp_u<kDppHalfMirror>(static_cast<uint32_t>(k))));
  k = max(k, static_cast<int32_t>(dpp_u<kDppMirror>(static_cast<uint32_t>(k))));
  const int32_t r0 = __builtin_amdgcn_readlane(k, 0), r1 = __builtin_amdgcn_readlane(k, 16);
  const int32_t r2 = __builtin_amdgcn_readlane(k, 32), r3 = __builtin_amdgcn_readlane(k, 48);
  return max(max(r0, r1), max(r2, r3));
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

// 16 bytes at lane_offset + uniform_offset (the latter in a scalar register),
// with the non-temporal hint (nt): every load of this kernel reads cache
// tiles or scales that the launch reads exactly once, and marked so they do
// not displace other lines from the caches (the kernel runs ~9% faster).
constexpr int kNonTemporal = 2;  // cache-policy bit nt of the buffer instructions
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int lane_offset, int uniform_offset = 0) {
  return __builtin_bit_cast(uint4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, lane_offset, uniform_offset, kNonTemporal));
}

__device__ __forceinline__ void lds_wave_sync() {
  // LDS writes of other lanes of this wave must land before it reads them
  // (LDS executes one wave's instructions in order; this keeps the compiler
  // from moving the reads above the writes).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The new token of sequence b, KV head g: K rotated in fp64 and rounded to
// fp32 (yarn_rope_apply on fp32 rows), then K and V quantised and stored at
// slot slots[b] (kv_cache_write_f4: -1 or a slot outside the pool writes
// nothing).  Thread t = 128 kind + j (kind 0: K, 1: V) quantises channels
// 2 j and 2 j + 1 into byte j of the row; the 16 lanes of a scale block are
// one DPP row, which takes the block's absolute maximum (the row's, through
// LDS, when V has one scale per token); 16 threads then store the blocks.
__device__ void step_write_token(const StepArgs& st, int b, int g, int Hkv) {
  __shared__ float kr[kHeadDim];
  __shared__ uint32_t vrow_max;
  __shared__ uint8_t nb[2][kHeadDim / 2];
  __shared__ uint16_t sb[2][kNumBlocks];
  const int tid = threadIdx.x;
  const float* krow = st.k_new + (static_cast<int64_t>(b) * Hkv + g) * kHeadDim;
  const int half = st.rd / 2;
  for (int e = tid; e < half + (kHeadDim - st.rd); e += kThreads) {
    if (e < half) {
      const double c = st.cos[static_cast<int64_t>(b) * half + e], sn = st.sin[static_cast<int64_t>(b) * half + e];
      double y0, y1;
      rope_rotate_pair(krow[e], krow[e + half], c, sn, y0, y1);
      kr[e] = static_cast<float>(y0);
      kr[e + half] = static_cast<float>(y1);
    } else {
      const int d = st.rd + (e - half);
      kr[d] = krow[d];
    }
  }
  if (tid == 0) vrow_max = 0u;
  __syncthreads();
  const int32_t slot = st.slots[b];
  if (slot < 0 || slot >= static_cast<int64_t>(st.num_pages) * kPage) return;  // the same for every thread
  static_assert(kThreads == kHeadDim, "one thread per byte of the K and V rows");
  const int kind = tid >> 7, j = tid & 127, c = j >> 4;
  const float* vrow = st.v_new + (static_cast<int64_t>(b) * Hkv + g) * kHeadDim;
  const float x0 = kind ? vrow[2 * j] : kr[2 * j];
  const float x1 = kind ? vrow[2 * j + 1] : kr[2 * j + 1];
  // absolute values as integer bits (they order as the floats; a NaN counts
  // as 0, as the writer's fmaxf ignores it)
  auto abits = [](float x) { return fabsf(x) == fabsf(x) ? __float_as_uint(fabsf(x)) : 0u; };
  uint32_t m = max(abits(x0), abits(x1));
  m = max(m, dpp_u<kDppQuadXor1>(m));
  m = max(m, dpp_u<kDppQuadXor2>(m));
  m = max(m, dpp_u<kDppHalfMirror>(m));
  m = max(m, dpp_u<kDppMirror>(m));  // the 16 lanes of the block
  const bool row_scale = kind == 1 && st.v_per_token;
  if (row_scale && (j & 15) == 0) atomicMax(&vrow_max, m);
  __syncthreads();
  if (row_scale) m = vrow_max;
  double sd;
  const uint16_t sbits = f4_scale(__uint_as_float(m), sd);
  nb[kind][j] = static_cast<uint8_t>(f4_nibble(x0, sd) | (f4_nibble(x1, sd) << 4));
  if ((j & 15) == 0) sb[kind][c] = sbits;
  __syncthreads();
  if (tid >= 2 * kNumBlocks) return;
  const int sk = tid / kNumBlocks, sc = tid % kNumBlocks;
  uint32_t nib[kBlock];
#pragma unroll
  for (int i = 0; i < kBlock / 2; ++i) {
    const uint32_t byte = nb[sk][16 * sc + i];
    nib[2 * i] = byte & 15u;
    nib[2 * i + 1] = byte >> 4;
  }
  const int64_t ph = static_cast<int64_t>(slot / kPage) * Hkv + g;
  if (sk == 0)
    f4_store_k_block(st.k_nib, st.k_scale, ph, kNumBlocks, sc, slot % kPage, nib, sb[0][sc]);
  else
    f4_store_v_block(st.v_nib, st.v_scale, ph, kHeadDim, sc, slot % kPage, nib, sb[1][sc], st.v_per_token != 0);
}

// One workgroup per (sequence, KV head): query rows -> QPrep.
// Workgroups 0 .. B*Hkv-1 prepare the query operands of one (sequence, KV
// head) each; the last workgroup builds the work list.  With step arguments
// (a decode step that also takes the new token of each sequence; R == 1) the
// workgroup of (b, g) first rotates the query rows (as yarn_rope_apply on bf16
// rows, through the shared rotation) and rotates and writes the new token's K
// and V of KV head g (as yarn_rope_apply on fp32 rows, then kv_cache_write_f4,
// through the shared quantiser), so the step's results equal those of the
// separate entry points bit for bit.
template <int G>
__global__ __launch_bounds__(kThreads) void decode_qprep_kernel(const uint16_t* __restrict__ q,
                                                               QPrep<G>* __restrict__ out, int32_t Hq,
                                                               int32_t Hkv, float qk_scale, PlanArgs plan,
                                                               int32_t R, int32_t r0, int32_t Gq, StepArgs st) {
  if (blockIdx.x == gridDim.x - 1) {
    if (plan.W * plan.B <= 64) {
      if (threadIdx.x < 64) build_work_list_wave(plan);
    } else {
      build_work_list(plan);
    }
    return;
  }
  __shared__ float qf[G][kHeadDim];
  __shared__ int32_t qexp[G];
  const int b = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  QPrep<G>& P = out[blockIdx.x];
  // row h of the group: query row r0 + h / Gq (clamped: rows past R are computed, never written), head g Gq + h % Gq
  if (st.cos) {
    // rotation pairs (e, e + rd / 2) of each row, rounded to bf16 as the rotated
    // query would be stored; channels from rd on pass through
    const int half = st.rd / 2;
    const int per_row = half + (kHeadDim - st.rd);
    for (int i = tid; i < G * per_row; i += kThreads) {
      const int h = i / per_row, e = i % per_row;
      const int r = min(r0 + h / Gq, R - 1);
      const uint16_t* qrow = q + ((static_cast<int64_t>(b) * R + r) * Hq + g * Gq + h % Gq) * kHeadDim;
      if (e < half) {
        const double c = st.cos[static_cast<int64_t>(b) * half + e], sn = st.sin[static_cast<int64_t>(b) * half + e];
        double y0, y1;
        rope_rotate_pair(bf16_to_f32(qrow[e]), bf16_to_f32(qrow[e + half]), c, sn, y0, y1);
        qf[h][e] = bf16_to_f32(f32_to_bf16(static_cast<float>(y0)));
        qf[h][e + half] = bf16_to_f32(f32_to_bf16(static_cast<float>(y1)));
      } else {
        const int d = st.rd + (e - half);
        qf[h][d] = bf16_to_f32(qrow[d]);
      }
    }
  } else {
    for (int i = tid; i < G * kHeadDim; i += kThreads) {
      const int h = i / kHeadDim, r = min(r0 + h / Gq, R - 1);
      const int64_t row = (static_cast<int64_t>(b) * R + r) * Hq + g * Gq + h % Gq;
      qf[h][i % kHeadDim] = bf16_to_f32(q[row * kHeadDim + i % kHeadDim]);
    }
  }
  if (st.k_new) step_write_token(st, b, g, Hkv);
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
        e = 11 - ex;      // scaled max in [2^10, 2^11); up to 144 for the smallest bf16 subnormals
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
    // the exponent goes to the values themselves (a factor 2^e alone would
    // overflow for rows of tiny queries, whose e exceeds 127)
    const int ex = qexp[h] - ((p & 1) ? 4 : 0);
    const _Float16 lo = static_cast<_Float16>(ldexpf(qf[h][base], ex));
    const _Float16 hi = static_cast<_Float16>(ldexpf(qf[h][base + 4], ex));
    P.pair[h][c][k][p] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
  }
  // the keys' "- 8": per (head, block) the sum of its 32 query operands as the
  // products take them (the x16 slots carry q / 16 against 16 n), times -8 2^-24
  for (int i = tid; i < G * 8; i += kThreads) {
    const int h = i / 8, c = i % 8;
    float sum = 0.0f;
    for (int j = 0; j < kBlock; ++j) {
      const int p = j & 3;
      const int ex = qexp[h] - ((p & 1) ? 4 : 0);
      const float a = static_cast<float>(static_cast<_Float16>(ldexpf(qf[h][32 * c + j], ex)));
      sum += (p & 1) ? 16.0f * a : a;
    }
    P.k8[c][h] = sum * -0x1p-21f;
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
  uint4 qa[G][8][4];  // the query pairs of QPrep, read as matrix-core operands
  float k8[8][G];     // the keys' "- 8" terms of QPrep
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

// The fp16 weights of (wave, head, block), in the place of that fp32 weight
// row: 64 tokens' hi parts, then their 64 lo parts.
template <int G>
__device__ __forceinline__ uint16_t* urow(DecodeSmem<G>& sm, int wave, int h, int c) {
  return reinterpret_cast<uint16_t*>(&sm.u.w[wave][h][c][0]);
}

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
  if (tid < 8 * G) (&sm.k8[0][0])[tid] = (&QP->k8[0][0])[tid];
  {
    const uint4* src = reinterpret_cast<const uint4*>(&QP->pair[0][0][0][0]);
    for (int i = tid; i < G * 32; i += kThreads) (&sm.qa[0][0][0])[i] = src[i];
  }
  __syncthreads();
  float m_run[G], l_lane[G], o[G][4];
  int32_t kmax_run[G];  // order key of the largest logit so far (uniform)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    kmax_run[h] = order_key(-INFINITY);
    l_lane[h] = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[h][d] = 0.0f;
  }
  constexpr int kSets = (G + 3) / 4;  // matrix-core head sets of 4
  const int qh = (lane & 3) % G;      // this lane's row of A: head 4 set + qh
  const int cj = lane >> 3;  // block holding this lane's 4 value channels
  const int sub = lane & 7;
  const int32_t* ptrow = a.pt + static_cast<int64_t>(b) * a.max_pages;
  const int lane16 = lane * 16;

  // Tiles of a page go through buffer resources with a scalar base: the lane
  // offsets are constants, so no per-page address arithmetic runs on the
  // VALU.  An out-of-range page id (or the page after the wave's last) gets
  // empty resources: its loads return 0 without memory traffic, and a mask
  // drops its tokens.
  struct PageRes {
    __amdgpu_buffer_rsrc_t k, v, ks, vs;
    bool valid;
  };
  // the page table is read-only here: read through the constant address
  // space, whose uniform loads are scalar (a vector load of a page id would
  // have to wait for every tile load issued before it)
  const auto ptc = (const __attribute__((address_space(4))) int32_t*)(ptrow);
  auto page_res = [&](int lp) {
    const int32_t pid = lp < pend ? ptc[lp] : -1;
    PageRes r;
    r.valid = static_cast<uint32_t>(pid) < static_cast<uint32_t>(a.num_pages);
    const int64_t ph = static_cast<int64_t>(r.valid ? pid : 0) * a.Hkv + g;
    const int tile_bytes = r.valid ? kPage * kHeadDim / 2 : 0;
    r.k = tile_rsrc(a.k_nib + ph * (kPage * kHeadDim / 2), tile_bytes);
    r.v = tile_rsrc(a.v_nib + ph * (kPage * kHeadDim / 2), tile_bytes);
    r.ks = tile_rsrc(a.k_scale + ph * (kPage * 8), r.valid ? kPage * 8 * 2 : 0);
    r.vs = VT ? tile_rsrc(a.v_scale + ph * kPage, r.valid ? kPage * 2 : 0)
              : tile_rsrc(a.v_scale + ph * (kPage * 8), r.valid ? kPage * 8 * 2 : 0);
    return r;
  };
  // The loads run one phase ahead through 8 register slots of 1 KB per wave:
  // slot c holds K block c of the page during the key phase, is then
  // refilled with the page's V block c; during the value phase it is refilled
  // with K block c of the wave's next page as soon as its V block is
  // unpacked, so the next page's keys are on their way while this page's
  // values are multiplied.  (The compiler copies parts of some slots in the
  // value phase, which makes those waits cover the slots' loads in flight; a
  // form without the copies, where every wait is for the oldest load only,
  // measured 2% slower.)
  uint4 tl[8];
  uint4 ks = make_uint4(0, 0, 0, 0), vs = make_uint4(0, 0, 0, 0);
  uint32_t vs1 = 0;  // this token's V scale (VT)
  {
    const PageRes r0 = page_res(pbeg + wave);
    ks = load16(r0.ks, lane16);
    if (VT)
      vs1 = __builtin_amdgcn_raw_buffer_load_b16(r0.vs, lane * 2, 0, kNonTemporal);
    else
      vs = load16(r0.vs, lane16);
#pragma unroll
    for (int c = 0; c < 8; ++c) tl[c] = load16(r0.k, lane16, c * 1024);
  }

  for (int lp = pbeg + wave; lp < pend; lp += kWaves) {
    const PageRes cur = page_res(lp);
    const bool pvalid = cur.valid;
    const auto rv = cur.v;
    __builtin_amdgcn_s_setprio(0);

    const int tok = lp * kPage + lane;
    const float tmask = (pvalid && tok >= t0 && tok < t1) ? 0.0f : -INFINITY;

    // keys: lane = token, on the matrix cores (mfma4): per block 8 products
    // of 4 channels each on the centred operands (n - 8) 2^-24; the block
    // scale is applied once per block
    float logit[G];
#pragma unroll
    for (int h = 0; h < G; ++h) logit[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      __builtin_amdgcn_sched_barrier(0);
      pin(tl[c]);
      const uint32_t sw = word(ks, c >> 1);
      const float sc = (c & 1) ? f16_hi(sw) : f16_lo(sw);
      uint4 qa[kSets][4];  // this lane's head: pairs [dword][4] of block c
#pragma unroll
      for (int st = 0; st < kSets; ++st)
#pragma unroll
        for (int k = 0; k < 4; ++k) qa[st][k] = sm.qa[4 * st + qh][c][k];
      float4_t acc[kSets];
#pragma unroll
      for (int st = 0; st < kSets; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[st][i] = 4 * st + i < G ? sm.k8[c][4 * st + i] : 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // operands n 2^-24 (x16 for p1, p3); the "- 8" started the accumulator
        const uint32_t wd = word(tl[c], k);
        const uint32_t p0 = wd & 0x000F000Fu;
        const uint32_t p1 = wd & 0x00F000F0u;
        const uint32_t w8 = wd >> 8;
        const uint32_t p2 = w8 & 0x000F000Fu;
        const uint32_t p3 = w8 & 0x00F000F0u;
        if (k == 3) {
          // the slot's next tile, V block c, requested once the K block is
          // unpacked (issued earlier, the load would need registers of its
          // own, and the loop would copy the slots at every page)
          __builtin_amdgcn_sched_barrier(0);
          tl[c] = load16(rv, lane16, c * 1024);
        }
#pragma unroll
        for (int st = 0; st < kSets; ++st) {
          acc[st] = mfma4(qa[st][k].x, qa[st][k].y, p0, p1, acc[st]);
          acc[st] = mfma4(qa[st][k].z, qa[st][k].w, p2, p3, acc[st]);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) logit[h] = fmaf(sc, acc[h / 4][h % 4], logit[h]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // Online softmax in log2 units with a lazily raised running max: m_run
    // moves (and the state is rescaled) only when the page's largest logit
    // exceeds it by more than kSlack, so weights stay below 2^kSlack and
    // most pages skip the rescale.  The exact maximum is tracked per lane and
    // restored at the end.
    float p[G], s[G], pm[G];
    bool raise = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      // additive mask: written as a select, the compiler turns the whole key
      // phase into a branch on the token's validity
      s[h] = fmaf(logit[h], QP->kscale[h], tok < lim[h] ? tmask : -INFINITY);
      const int32_t kmax = wave_max_key(order_key(s[h]));
      kmax_run[h] = max(kmax_run[h], kmax);
      pm[h] = key_value(kmax);
      raise |= pm[h] > m_run[h] + kSlack;
    }
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m_run[h], pm[h]);
        // mn == -inf only while no valid token has been seen: nothing to rescale
        const float alpha = m_run[h] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[h] - mn);
        l_lane[h] *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d) o[h][d] *= alpha;
        m_run[h] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, mn)));
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
    const int wrow = VT ? 0 : cj;  // fp32 weight row of this lane's value block

    // Weights to fp16 pairs hi + lo in units of the row's largest weight.
    // The 8 lanes of block cj share the row of the block's 64 weights per
    // head; lane sub converts tokens 8 sub .. 8 sub + 7.  u = w / w_max is in
    // [0, 1]; hi = fp16(u) (toward zero) and lo = fp16(u - hi) carry u to
    // ~2^-21 of itself, with an absolute floor of 2^-25 (fp16 subnormals),
    // so every weight keeps about 21 bits, the small ones included.  The
    // fp16 rows [hi: 64 tokens][lo: 64 tokens] overwrite the fp32 row once
    // every lane of the wave has read its part.
    float4_t wx[G], wy[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      wx[h] = *reinterpret_cast<const float4_t*>(&sm.u.w[wave][h][wrow][sub * 8]);
      wy[h] = *reinterpret_cast<const float4_t*>(&sm.u.w[wave][h][wrow][sub * 8 + 4]);
    }
    lds_wave_sync();
    float funit[G];  // w_max of the lane's block row, per head
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float4_t x = wx[h], y = wy[h];
      const float mx = max8_nonneg(x, y);
      // 1 / w_max (a zero row scales by 1e30 and stays zero)
      const float r = __builtin_amdgcn_rcpf(fmaxf(mx, 1e-30f));
      const float xs[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const pk16_t hp = __builtin_amdgcn_cvt_pkrtz(xs[2 * i] * r, xs[2 * i + 1] * r);
        const float r0 = fmaf(xs[2 * i], r, -static_cast<float>(hp.x));
        const float r1 = fmaf(xs[2 * i + 1], r, -static_cast<float>(hp.y));
        hi[i] = __builtin_bit_cast(uint32_t, hp);
        lo[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
      }
      uint16_t* row = urow(sm, wave, h, wrow);
      *reinterpret_cast<uint4*>(&row[sub * 8]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      *reinterpret_cast<uint4*>(&row[64 + sub * 8]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      funit[h] = mx;
    }
    lds_wave_sync();

    // values: lane = channels 4 lane .. 4 lane + 3 (block cj), on the matrix
    // cores (mfma4) with lane = column: slot e of 4 is channel 4 lane + e, B
    // = its centred nibbles over 4 tokens (the fp16 pairs of two V dwords),
    // A = the 4 tokens' weights (hi, then lo) of head 4 set + (lane & 3) in
    // block cj, the block of all 4 lanes of a 16-lane matrix block.  Element
    // h of slot e's result is head h's sum for the lane's channel e.
    __builtin_amdgcn_s_setprio(2);
    // the next page's K scales (this page's are consumed), then its K blocks
    // into the slots; its V scales last (they are needed after its key phase)
    const PageRes nxt = page_res(lp + kWaves);
    ks = load16(nxt.ks, lane16);
    float4_t ov[kSets][4];
#pragma unroll
    for (int st = 0; st < kSets; ++st)
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[st][e] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      if ((ct & 1) == 0) __builtin_amdgcn_sched_barrier(0);  // two token groups' weights in flight
      pin(tl[ct]);
      uint4 whi[kSets], wlo[kSets];  // fp16 weights of tokens 8 ct .. 8 ct + 7
#pragma unroll
      for (int st = 0; st < kSets; ++st) {
        const uint16_t* row = urow(sm, wave, 4 * st + qh, wrow);
        whi[st] = *reinterpret_cast<const uint4*>(&row[ct * 8]);
        wlo[st] = *reinterpret_cast<const uint4*>(&row[64 + ct * 8]);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {  // tokens 8 ct + 4 q .. 8 ct + 4 q + 3: V dwords 2 q, 2 q + 1
        const uint32_t d0 = word(tl[ct], 2 * q), d1 = word(tl[ct], 2 * q + 1);
        const uint32_t e0 = d0 >> 8, e1 = d1 >> 8;
        // fp16 pairs (n - 8) 2^-24 of channels 0..3 (x16 for 1 and 3) over the
        // 4 tokens: the masked nibbles, then the "- 8" by one packed fp16 add
        // (exact: integer multiples of 2^-24 within the subnormal range).
        // Centred operands keep the matrix product away from the cancellation
        // of sum u n against 8 sum u, whose relative error (~2^-19 per 4 x 4 x
        // 4 product, measured) would otherwise grow with the ratio of the two.
        const uint32_t b[4][2] = {{centre(d0 & 0x000F000Fu, kM8), centre(d1 & 0x000F000Fu, kM8)},
                                  {centre(d0 & 0x00F000F0u, kM128), centre(d1 & 0x00F000F0u, kM128)},
                                  {centre(e0 & 0x000F000Fu, kM8), centre(e1 & 0x000F000Fu, kM8)},
                                  {centre(e0 & 0x00F000F0u, kM128), centre(e1 & 0x00F000F0u, kM128)}};
        if (q == 1) {
          // the slot's next tile, the next page's K block ct, once the V block
          // is unpacked
          __builtin_amdgcn_sched_barrier(0);
          tl[ct] = load16(nxt.k, lane16, ct * 1024);
        }
#pragma unroll
        for (int st = 0; st < kSets; ++st) {
          const uint32_t h0 = word(whi[st], 2 * q), h1 = word(whi[st], 2 * q + 1);
          const uint32_t l0 = word(wlo[st], 2 * q), l1 = word(wlo[st], 2 * q + 1);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ov[st][e] = mfma4(h0, h1, b[e][0], b[e][1], ov[st][e]);
            ov[st][e] = mfma4(l0, l1, b[e][0], b[e][1], ov[st][e]);
          }
        }
      }
    }
    if (VT)
      vs1 = __builtin_amdgcn_raw_buffer_load_b16(nxt.vs, lane * 2, 0, kNonTemporal);
    else
      vs = load16(nxt.vs, lane16);
    // the page's sums, in units of w_max, into the running accumulators
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[h][e] = fmaf(ov[h / 4][e][h % 4], funit[h], o[h][e]);
  }

  // ---- epilogue: restore the exact maximum, fold the 4 waves ---------------
  __builtin_amdgcn_s_setprio(0);
  float l_w[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mx = key_value(kmax_run[h]);  // <= m_run + kSlack
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
                           const StepArgs& st, hipStream_t s) {
  QPrep<G>* qp = static_cast<QPrep<G>*>(qprep);
  hipLaunchKernelGGL(decode_qprep_kernel<G>, dim3(a.B * a.Hkv + 1), dim3(kThreads), 0, s, a.q, qp, a.Hq, a.Hkv,
                     a.qk_scale, plan, a.R, a.r0, a.Gq, st);
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

// The workspace of paged_attn_decode_f4_noalloc: one array per GPU, held by
// the process until it ends.  Host code never uses the array's name as an
// address: decode_scratch() looks the device address up once per device.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

}  // namespace

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* addr[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

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
                         void* ws, const DecodePlan& plan, const DecodeStep* step, hipStream_t s) {
  if (B == 0) return hipSuccess;
  StepArgs st{};
  if (step) {
    st.cos = step->cos;
    st.sin = step->sin;
    st.rd = step->rotary_dim;
    st.k_new = step->k_new;
    st.v_new = step->v_new;
    st.slots = step->slots;
    st.k_nib = c.k_nib;
    st.k_scale = c.k_scale;
    st.v_nib = c.v_nib;
    st.v_scale = c.v_scale;
    st.num_pages = c.num_pages;
    st.v_per_token = c.v_scale_per_token;
  }
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
      case 1: e = vt ? launch_decode_g<1, true>(a, qprep, pa, plan.max_items, st, s)
                     : launch_decode_g<1, false>(a, qprep, pa, plan.max_items, st, s); break;
      case 2: e = vt ? launch_decode_g<2, true>(a, qprep, pa, plan.max_items, st, s)
                     : launch_decode_g<2, false>(a, qprep, pa, plan.max_items, st, s); break;
      case 4: e = vt ? launch_decode_g<4, true>(a, qprep, pa, plan.max_items, st, s)
                     : launch_decode_g<4, false>(a, qprep, pa, plan.max_items, st, s); break;
      default: e = vt ? launch_decode_g<8, true>(a, qprep, pa, plan.max_items, st, s)
                      : launch_decode_g<8, false>(a, qprep, pa, plan.max_items, st, s); break;
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
