// paged_attn_prefill_f4_fp8: the prompt chunk's causal attention with 8-bit products.
//
// What is computed (ignis configuration page, context-and-speculation, the
// --model-prefill-attention row: an 8-bit precision for the prompt attention
// over a 4-bit-cache chunk, the scores Q.K^T in INT8 and the weighted sum P.V
// in E4M3): the attention of paged_attn_prefill_f4 with these roundings, for
// query row r at position p over cache tokens [0, p]:
//  * the query row to INT8 with one power-of-two scale sigma = 2^(e - 7),
//    max |q| < 2^e, round half to even, clamped to +-127;
//  * each cached key to INT8 with one power-of-two scale per token, tau =
//    2^(E - 4), E = (fp16 exponent field of the token's largest block scale) -
//    14, the value c s / tau rounded to nearest, ties to even (always within
//    [-128, 112]);
//  * scores in log2 units x = S sigma tau qk, S the exact INT8 dot product and
//    qk = sm_scale log2(e) in fp32;
//  * weights to E4M3 per 32-token group of a row: G = ceil(max x of the group),
//    P8 = e4m3(2^(x - G)), the group's weights carrying 2^G;
//  * values to E4M3 per 32-token group and 32-channel block: F = (fp16
//    exponent field of the largest V scale there) - 19, V8 = e4m3(c s 2^-F);
//  * out = sum P8 2^G V8 2^F / sum 2^x (the unquantised weights below).
//
// Shape of the work: a workgroup of 8 waves owns 64 query positions of one KV
// head (256 rows once the 4 query heads of the group are stacked, 32 per wave,
// one lane per row; 8 positions per wave as in the fp16 prefill) and a range
// of key pages.  With 8 waves sharing a page's conversion each thread converts
// one 16-byte unit of keys and one of values per page; two waves per SIMD
// hide each other's latencies.  Per page of 64 keys:
//  1. the workgroup requantises the page's keys into LDS as INT8 [token]
//     [channel] (one packed fp16 FMA per pair of values) and its values as
//     E4M3 V^T [channel][token];
//  2. each wave forms S^T = K Q^T with the INT8 matrix core
//     (v_mfma_i32_32x32x32_i8: exact integer sums), 8 per 32-token tile;
//  3. the softmax runs lane-local in log2 units with a lazily raised running
//     max (an integer, so the rescale is exact); the weights of each 32-token
//     group are rounded to E4M3 in the lanes that hold them;
//  4. O^T += V^T P^T with the block-scaled FP8 matrix core
//     (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3, fp32 accumulate): one
//     instruction per 32 channels covers the page's 64 tokens as two k-blocks,
//     each with its own E8M0 scales, 2^F for the values (per channel row) and
//     2^(G - m) for the weights (per query row), so neither operand is
//     rescaled in registers.
// The value rows in LDS hold channel 4 j + c at row 64 c + j, so the 64 lanes
// that convert the 64 channel quads of a token group write 64 consecutive
// rows; the output is written back in channel order.
#include "f4kv_internal.h"

namespace f4kv {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kQPos = 64;               // query positions per workgroup (8 per wave)
constexpr int kKRow = kHeadDim + 16;    // bytes per INT8 key row in LDS
constexpr int kVRow = kPage + 8;        // bytes per E4M3 value row in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.0f;  // log2 units a group maximum may exceed the running max by

struct Fp8Args {
  const uint8_t* k_nib;
  const uint16_t* k_scale;
  const uint8_t* v_nib;
  const uint16_t* v_scale;
  const uint16_t* q;
  const int32_t* pt;
  float* o;  // [S][R][D], R = T * Hq
  float* m;  // [S][R] or null
  float* l;
  int32_t T, Hq, Hkv, num_pages, pos0;
  int32_t kv_splits;
  float qk_scale;  // sm_scale * log2(e), fp32
};

struct __align__(16) Fp8Smem {
  uint8_t kt[kPage][kKRow];         // keys, INT8 [token][channel in unpack order]
  uint8_t vt[kHeadDim][kVRow];      // values, E4M3 [64 c + j for channel 4 j + c][token in MFMA order]
  float tau[kPage];                 // the INT8 key scale of each token
  uint16_t vsc[2][8][kPage];        // V scales [page parity][block][token] (one scale per token: row 0)
  uint32_t vmax[2][2][8];           // largest V scale bits [page parity][token group][block]
  i32x4 qs[kWaves][8][64];          // INT8 query operands [wave][score step][lane]
};

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Raw cells of one page for this thread.  Keys: the unit (block w, token t)
// (w = wave, t = lane) and the token's eight K scales; threads below 256 also
// hold one dword of the V scale tile (token tid / 4, blocks 2 (tid % 4), + 1;
// with one V scale per token, threads below 32 hold tokens 2 tid, + 1).
// Values: the unit (token group w of 8 tokens, channel quad t).
struct KRaw {
  uint4 k;
  uint4 ks;      // the eight K block scales of token t
  uint32_t vsd;  // two V scales
};
struct VRaw {
  uint4 v;
};

template <bool VT>
__device__ __forceinline__ void load_k(const Fp8Args& a, int64_t ph, int tid, KRaw& r) {
  const uint4* kt = reinterpret_cast<const uint4*>(a.k_nib + ph * (kPage * kHeadDim / 2));
  const int w = tid >> 6, t = tid & 63;
  r.k = kt[w * 64 + t];
  r.ks = reinterpret_cast<const uint4*>(a.k_scale + ph * (kPage * 8))[t];
  if (VT)
    r.vsd = reinterpret_cast<const uint32_t*>(a.v_scale + ph * kPage)[tid & 31];
  else
    r.vsd = reinterpret_cast<const uint32_t*>(a.v_scale + ph * (kPage * 8))[tid & 255];
}

__device__ __forceinline__ void load_v(const Fp8Args& a, int64_t ph, int tid, VRaw& r) {
  const uint4* vt = reinterpret_cast<const uint4*>(a.v_nib + ph * (kPage * kHeadDim / 2));
  r.v = vt[tid];
}

// The V scales of the page to LDS ([block][token]) and their largest value per
// (token group, block) into vmax (fp16 bits of non-negative scales order as
// unsigned integers).
template <bool VT>
__device__ __forceinline__ void stage_vscales(Fp8Smem& sm, const KRaw& r, int tid, int parity) {
  if (VT) {
    if (tid < 32) {
      *reinterpret_cast<uint32_t*>(&sm.vsc[parity][0][2 * tid]) = r.vsd;
      const uint32_t mx = max(r.vsd & 0xFFFFu, r.vsd >> 16);
      atomicMax(&sm.vmax[parity][tid >> 4][0], mx);
    }
  } else if (tid < 256) {
    const int t = tid >> 2, b = 2 * (tid & 3);
    sm.vsc[parity][b][t] = static_cast<uint16_t>(r.vsd);
    sm.vsc[parity][b + 1][t] = static_cast<uint16_t>(r.vsd >> 16);
    atomicMax(&sm.vmax[parity][t >> 5][b], r.vsd & 0xFFFFu);
    atomicMax(&sm.vmax[parity][t >> 5][b + 1], r.vsd >> 16);
  }
}

// Keys of this thread's unit to INT8.  With the block scale s = M 2^(max(e5, 1) - 25) (M
// its significand, e5 its exponent field) and tau = 2^(e5max - 18), c s / tau
// = c M 2^-k for k = e5max + 7 - max(e5, 1) >= 6, and |c M 2^-k| <= 256.
// Rounded to nearest, ties to even, in one packed fp16 FMA per pair of values:
// fma(c, M 2^-k, 1536) is exact before its single rounding, and fp16 values in
// [1024, 2048) are the integers, so the result is 1536 + rne(c M 2^-k) (1536
// is even, so a tie lands on the even integer); its low byte is that integer
// as an INT8 (1536 = 6 x 256).  c = n - 8 comes exactly out of 1024 + n (the
// nibble ORed into the mantissa of 1024) minus 1032.  M 2^-k is exact in fp16
// for k <= 14; for k >= 15 every |c M 2^-k| < 1/2, so the code is 0 whatever
// the rounding of M 2^-k.  Nibble pairs (j, j + 4) of a dword come out of one
// AND-OR; the bytes are stored as channels 0, 1, 4, 5, 2, 3, 6, 7 of each group
// of 8, and the query operands use the same order.
// tau goes to LDS with the sign of the logit scale, so that the scores up to
// the positive factor |sigma qk| order like the scores themselves.
typedef _Float16 half2v_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void unpack_k(Fp8Smem& sm, const KRaw& r, int tid, float tau_sign, uint32_t magic) {
  const int c = tid >> 6, t = tid & 63;
  const uint32_t b01 = word(r.ks, 0), b23 = word(r.ks, 1), b45 = word(r.ks, 2), b67 = word(r.ks, 3);
  // largest of the eight scales (non-negative fp16 bits compare as integers)
  const uint32_t m1 = max(max(b01 & 0xFFFFu, b01 >> 16), max(b23 & 0xFFFFu, b23 >> 16));
  const uint32_t m2 = max(max(b45 & 0xFFFFu, b45 >> 16), max(b67 & 0xFFFFu, b67 >> 16));
  const int e5max = static_cast<int>(max(m1, m2) >> 10);
  const uint32_t sb = (word(r.ks, c >> 1) >> (16 * (c & 1))) & 0xFFFFu;
  const int e5 = static_cast<int>(sb >> 10);
  const int M = static_cast<int>(sb & 1023u) | (e5 ? 1024 : 0);
  const int k = e5max + 7 - max(e5, 1);
  const _Float16 S = static_cast<_Float16>(__builtin_amdgcn_ldexpf(static_cast<float>(M), -k));
  const half2v_t Sv = {S, S};
  const half2v_t off = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
  const half2v_t bias = {static_cast<_Float16>(1536.0f), static_cast<_Float16>(1536.0f)};
  uint32_t out[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w = word(r.k, d);
    uint32_t p[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const half2v_t cn = __builtin_bit_cast(half2v_t, ((w >> (4 * s)) & 0x000F000Fu) | magic) + off;  // n - 8
      p[s] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(cn, Sv, bias));
    }
    // bytes 0 and 2 of each 16-bit pair: channels (0, 1, 4, 5) and (2, 3, 6, 7)
    out[2 * d] = __builtin_amdgcn_perm(p[1], p[0], 0x06020400u);
    out[2 * d + 1] = __builtin_amdgcn_perm(p[3], p[2], 0x06020400u);
  }
  uint4* dst = reinterpret_cast<uint4*>(&sm.kt[t][32 * c]);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  if (tid < 64) sm.tau[t] = __builtin_amdgcn_ldexpf(tau_sign, e5max - 18);
}

// Values of this thread's unit (tokens 8 w .., channel quad j = lane) to E4M3.  The
// 8 tokens of the unit fall in one 32-token group g and one 8-token column a
// of it; within a group the MFMA takes tokens 8 a + 4 h + i from lane half h,
// byte 4 a + i, so each channel gets two 4-byte pieces (h = 0, 1).
// byte b of w as a float (v_cvt_f32_ubyte<b>)
__device__ __forceinline__ float byte_to_f32(uint32_t w, int b) { return static_cast<float>((w >> (8 * b)) & 0xFFu); }

template <bool VT>
__device__ __forceinline__ void unpack_v(Fp8Smem& sm, const VRaw& r, int tid, int parity) {
  const int c8 = tid >> 6, j = tid & 63;
  const int g = c8 >> 2, acol = c8 & 3, blk = j >> 3;
  const uint32_t mx = sm.vmax[parity][g][VT ? 0 : blk];
  const float inv = __builtin_amdgcn_ldexpf(1.0f, 19 - static_cast<int>(mx >> 10));  // 2^-F
  const uint4 s4 = *reinterpret_cast<const uint4*>(&sm.vsc[parity][VT ? 0 : blk][8 * c8]);
  float sv[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = word(s4, i);
    sv[2 * i] = f16bits_to_f32(static_cast<uint16_t>(w)) * inv;
    sv[2 * i + 1] = f16bits_to_f32(static_cast<uint16_t>(w >> 16)) * inv;
  }
  // x[token][channel]: dword k holds tokens 2k, 2k+1; byte 2r + q: channels 2q (low), 2q + 1 (high)
  float x[8][4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = word(r.v, k);
    // one nibble per byte, converted by byte (v_cvt_f32_ubyte0..3)
    uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    // opaque to the optimiser, which would otherwise extract each nibble by itself
    asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int tk = 2 * k + rr;
      const float s = sv[tk], z = -8.0f * sv[tk];
      x[tk][0] = fmaf(byte_to_f32(lo, 2 * rr), s, z);
      x[tk][1] = fmaf(byte_to_f32(hi, 2 * rr), s, z);
      x[tk][2] = fmaf(byte_to_f32(lo, 2 * rr + 1), s, z);
      x[tk][3] = fmaf(byte_to_f32(hi, 2 * rr + 1), s, z);
    }
  }
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    uint8_t* row = &sm.vt[64 * ch + j][0];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int d = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * h][ch], x[4 * h + 1][ch], 0, false);
      d = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * h + 2][ch], x[4 * h + 3][ch], d, true);
      *reinterpret_cast<int*>(row + 32 * h + 16 * g + 4 * acol) = d;
    }
  }
}

template <bool VT>
__global__ __launch_bounds__(kThreads, 1) void prefill_fp8_kernel(Fp8Args a, const int32_t* __restrict__ pt) {
  __shared__ Fp8Smem sm;
  const int qt = blockIdx.x;     // query tile
  const int g = blockIdx.y;      // KV head
  const int split = blockIdx.z;  // key-range split
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;

  // this lane's query row: position qt * 64 + wave * 8 + col / 4, head g * 4 + col % 4
  const int qi = qt * kQPos + wave * 8 + col / 4;
  const bool qvalid = qi < a.T;
  const int qpos = a.pos0 + qi;
  const int hq = g * 4 + (col & 3);
  const int qpos_first = a.pos0 + qt * kQPos;  // no key below it needs a mask

  const int tile_last = min(a.T, (qt + 1) * kQPos) - 1;
  const int npages = (a.pos0 + tile_last) / kPage + 1;
  const int per = (npages + a.kv_splits - 1) / a.kv_splits;
  const int pbeg = __builtin_amdgcn_readfirstlane(split * per);
  const int pend = __builtin_amdgcn_readfirstlane(min(npages, pbeg + per));

  // ---- query row to INT8: B operands of the 8 score steps (channels 32 s + 16 half .. + 15), kept in LDS ----
  float row_scale;  // |sigma qk|
  {
    const uint16_t* qrow = a.q + (static_cast<int64_t>(qvalid ? qi : 0) * a.Hq + hq) * kHeadDim;
    float qv[8][16];
    float mx = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint4* src = reinterpret_cast<const uint4*>(qrow + 32 * s + 16 * half);
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const uint4 raw = src[v];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = word(raw, i);
          qv[s][8 * v + 2 * i] = bf16_to_f32(static_cast<uint16_t>(w));
          qv[s][8 * v + 2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w >> 16));
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(qv[s][i]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    int e = 7;  // an all-zero row: sigma = 1
    if (mx > 0.0f) frexpf(mx, &e);  // mx < 2^e
    const float inv_sigma = __builtin_amdgcn_ldexpf(1.0f, 7 - e);
    // (a zero logit scale: tau is 0 below, every score 0)
    row_scale = a.qk_scale == 0.0f ? 1.0f : __builtin_amdgcn_ldexpf(fabsf(a.qk_scale), e - 7);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      int b[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float r = fminf(fmaxf(__builtin_rintf(qv[s][i] * inv_sigma), -127.0f), 127.0f);
        b[i] = static_cast<int>(r) & 0xFF;
      }
      // each group of 8 channels in the order 0, 1, 4, 5, 2, 3, 6, 7
      i32x4 op;
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int* c = b + 8 * v;
        op[2 * v] = c[0] | (c[1] << 8) | (c[4] << 16) | (c[5] << 24);
        op[2 * v + 1] = c[2] | (c[3] << 8) | (c[6] << 16) | (c[7] << 24);
      }
      sm.qs[wave][s][lane] = op;
    }
  }

  const float tau_sign = a.qk_scale > 0.0f ? 1.0f : (a.qk_scale < 0.0f ? -1.0f : 0.0f);
  uint32_t nmagic = 0x64006400u;  // fp16 1024 in both halves, kept in a VGPR (one literal per instruction)
  asm volatile("" : "+v"(nmagic));
  f32x16 acc[8];  // O^T: 8 tiles of 32 value rows (rows 32 ct .. of the LDS order)
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] = f32x16{};
  float m_run = -INFINITY;  // an integer once finite
  float s_max = -INFINITY, l_lane = 0.0f;

  auto page_handle = [&](int lp, bool& valid) {
    const int32_t pid = pt[lp];
    valid = static_cast<uint32_t>(pid) < static_cast<uint32_t>(a.num_pages);
    return static_cast<int64_t>(valid ? pid : 0) * a.Hkv + g;
  };

  if (tid < 32) reinterpret_cast<uint32_t*>(sm.vmax)[tid] = 0u;
  __syncthreads();

  // cells in flight: vcur = V of page lp; requested at the top of iteration
  // lp: K and V of page lp + 1 (the keys are converted in this iteration's
  // second half, the values in the next iteration)
  KRaw kraw{};
  VRaw vcur{}, vnext{};
  bool cur_valid = false, next_valid = false;
  if (pbeg < pend) {
    const int64_t ph0 = page_handle(pbeg, cur_valid);
    load_k<VT>(a, ph0, tid, kraw);
    load_v(a, ph0, tid, vcur);
    unpack_k(sm, kraw, tid, tau_sign, nmagic);
    stage_vscales<VT>(sm, kraw, tid, pbeg & 1);
  }

  for (int lp = pbeg; lp < pend; ++lp) {
    const int par = lp & 1;
    if (lp + 1 < pend) {
      const int64_t ph1 = page_handle(lp + 1, next_valid);
      load_k<VT>(a, ph1, tid, kraw);
      load_v(a, ph1, tid, vnext);
    }
    __syncthreads();  // keys and V scales of this page are in LDS; every wave is done with the previous values

    // ---- values of this page to E4M3 (read in the PV step below) ----
    if (tid < 16) sm.vmax[par ^ 1][tid >> 3][tid & 7] = 0u;  // the next page's maxima start from 0
    unpack_v<VT>(sm, vcur, tid, par);

    // ---- S^T = K Q^T for both 32-token tiles, exact in INT32 ----
    i32x16 st[2] = {i32x16{}, i32x16{}};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const i32x4 qop = sm.qs[wave][s][lane];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const i32x4 kop = *reinterpret_cast<const i32x4*>(&sm.kt[32 * tt + col][32 * s + 16 * half]);
        st[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop, qop, st[tt], 0, 0, 0);
      }
    }
    float x[2][16];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      // rows 8 q + 4 half + i of the tile: x = S tau with the token scales from LDS; the
      // scores in log2 units are x row_scale (row_scale > 0, the sign is in tau)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4_t tau4 = *reinterpret_cast<const float4_t*>(&sm.tau[32 * tt + 8 * q4 + 4 * half]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[tt][4 * q4 + i] = static_cast<float>(st[tt][4 * q4 + i]) * tau4[i];  // exact: tau is a power of two
      }
    }

    // ---- softmax: mask, group maxima, lazy raise of the running max ----
    // (the mask only on pages that reach past the tile's first position: a
    // branch of its own, which keeps its compares off the other pages)
    const bool need_mask = !cur_valid || lp * kPage + 63 > qpos_first;
    if (need_mask) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int tok = lp * kPage + 32 * tt + 8 * (e >> 2) + 4 * half + (e & 3);
          // in place: the unmasked pages keep the scores where they are
          asm volatile("" : "+v"(x[tt][e]));
          if (!(cur_valid && qvalid && tok <= qpos)) x[tt][e] = -INFINITY;
          asm volatile("" : "+v"(x[tt][e]));
        }
    }
    float gmax[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float mx = x[tt][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, x[tt][e]);
      gmax[tt] = mx;
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) gmax[tt] = fmaxf(gmax[tt], __shfl_xor(gmax[tt], 32, 64)) * row_scale;
    s_max = fmaxf(s_max, fmaxf(gmax[0], gmax[1]));
    const float G0 = ceilf(gmax[0]), G1 = ceilf(gmax[1]);  // -inf stays -inf
    const float pmax = fmaxf(G0, G1);
    const bool raise = pmax > m_run + kSlack;
    if (__ballot(raise)) {
      const float mn = raise ? pmax : m_run;
      const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, static_cast<int>(m_run - mn));
      m_run = mn;
      l_lane *= alpha;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] *= alpha;
    }

    // ---- weights to E4M3, group by group; B operand bytes 0-15 tile 0, 16-31 tile 1 ----
    i32x8 pop;
    int scb[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const float G = tt ? G1 : G0;
      const bool live = G != -INFINITY;
      const float off = live ? G : 0.0f;
      float e[16], psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        e[i] = __builtin_amdgcn_exp2f(fmaf(x[tt][i], row_scale, -off));  // 0 for masked keys
        psum += e[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int d = __builtin_amdgcn_cvt_pk_fp8_f32(e[4 * i], e[4 * i + 1], 0, false);
        pop[4 * tt + i] = __builtin_amdgcn_cvt_pk_fp8_f32(e[4 * i + 2], e[4 * i + 3], d, true);
      }
      const int sh = live ? static_cast<int>(G - m_run) : 0;  // <= kSlack
      l_lane += live ? __builtin_amdgcn_ldexpf(psum, sh) : 0.0f;
      scb[tt] = max(sh + 127, 0);  // E8M0; below 2^-127 the group's weight is negligible
    }
    const int scale_b = half ? scb[1] : scb[0];

    __syncthreads();  // values of this page are in LDS; every wave is done with this page's keys

    // ---- keys of the next page to INT8 and its V scales, while the matrix cores work on P.V ----
    if (lp + 1 < pend) {
      unpack_k(sm, kraw, tid, tau_sign, nmagic);
      stage_vscales<VT>(sm, kraw, tid, par ^ 1);
    }

    // ---- O^T += V^T P^T: one block-scaled FP8 MFMA per 32 value rows ----
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const int vrow = 32 * ct + col;  // channel 4 (vrow % 64) + vrow / 64
      const uint8_t* src = &sm.vt[vrow][32 * half];
      i32x8 vop;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint2 w = *reinterpret_cast<const uint2*>(src + 8 * i);
        vop[2 * i] = static_cast<int>(w.x);
        vop[2 * i + 1] = static_cast<int>(w.y);
      }
      const int blk = VT ? 0 : ((vrow & 63) >> 3);
      const int scale_a = static_cast<int>(sm.vmax[par][half][blk] >> 10) - 19 + 127;  // 2^F of token group `half`
      acc[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, pop, acc[ct], 0, 0, 0, scale_a, 0, scale_b);
    }

    vcur = vnext;
    cur_valid = next_valid;
  }

  // ---- epilogue ----
  const float f = s_max == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - s_max);
  const float Lr = l_lane + __shfl_xor(l_lane, 32, 64);  // in units of 2^m_run
  const float L = Lr * f;
  if (!qvalid) return;
  const int64_t R = static_cast<int64_t>(a.T) * a.Hq;
  const int64_t row = static_cast<int64_t>(split) * R + static_cast<int64_t>(qi) * a.Hq + hq;
  const float inv = Lr > 0.0f ? 1.0f / Lr : 0.0f;
  float* dst = a.o + row * kHeadDim;
  // element e of tile ct is value row 32 ct + 8 (e / 4) + 4 half + e % 4, i.e. channel
  // 4 (32 (ct % 2) + r) + ct / 2: tiles 0, 2, 4, 6 give channels 4 r .. 4 r + 3
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int r = 8 * (e >> 2) + 4 * half + (e & 3);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      float4_t v;
      v.x = acc[hi + 0][e] * inv;
      v.y = acc[hi + 2][e] * inv;
      v.z = acc[hi + 4][e] * inv;
      v.w = acc[hi + 6][e] * inv;
      *reinterpret_cast<float4_t*>(dst + 4 * (32 * hi + r)) = v;
    }
  }
  if (half == 0) {
    if (a.m) a.m[row] = L > 0.0f ? s_max * kLn2 : -INFINITY;
    if (a.l) a.l[row] = L;
  }
}

}  // namespace

hipError_t launch_prefill_fp8(const f4kv_cache& c, const uint16_t* q, const int32_t* pt, int32_t max_pages,
                              int32_t T, int32_t Hq, int32_t pos0, float sm_scale, float* out, float* out_m,
                              float* out_l, void* ws, const PrefillPlan& plan, hipStream_t s) {
  (void)max_pages;
  if (T == 0) return hipSuccess;
  Fp8Args a;
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
  const dim3 grid(plan.q_tiles, a.Hkv, plan.kv_splits);
  timing_begin(F4KV_KERNEL_PREFILL_FP8, s);
  if (c.v_scale_per_token)
    hipLaunchKernelGGL(prefill_fp8_kernel<true>, grid, dim3(kThreads), 0, s, a, pt);
  else
    hipLaunchKernelGGL(prefill_fp8_kernel<false>, grid, dim3(kThreads), 0, s, a, pt);
  hipError_t e = hipGetLastError();
  timing_end(F4KV_KERNEL_PREFILL_FP8, s);
  if (e != hipSuccess || plan.kv_splits == 1) return e;
  return launch_merge(pm, pl, a.o, plan.kv_splits, static_cast<int32_t>(R), kHeadDim, out, out_m, out_l, s);
}

}  // namespace f4kv
