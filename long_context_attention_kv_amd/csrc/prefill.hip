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
//     exact pair hi + lo: the block scale s is split into s_hi (its top 8
//     significant bits) and s_lo = s - s_hi, so (n - 8) * s_hi and
//     (n - 8) * s_lo are both exact in fp16 and the dequantisation runs on
//     packed fp16 arithmetic (two values per instruction).  A single fp16
//     rounding of the dequantised keys alone would move the output by up to
//     ~2e-3 of its RMS, and of V or P by ~1e-3 each;
//  2. each wave forms S^T = K Q^T for its 32 query rows with fp16 MFMA
//     (v_mfma_f32_32x32x16_f16, fp32 accumulate) as K_hi Q + K_lo Q, so one
//     lane owns one query row and its row max / sum are mostly lane-local;
//  3. online softmax in log2 units with a lazily raised running max; the
//     causal mask only on pages that reach past the tile's first position;
//  4. O^T += V^T P^T with the same MFMA as V_hi P_hi + V_hi P_lo + V_lo P,
//     P split into fp16 hi + lo like V, so only fp32 rounding remains.
//     The exp'd scores already sit in the B-operand lanes; the token order
//     inside a k-step is permuted to match and the V^T reads use the same
//     permutation.
// The dequantisation overlaps the matrix work of the other operand: V of a
// page is unpacked while the waves multiply its K, and K of the next page
// while they multiply V (two barriers per page).  The raw cells of the next
// page are requested a page ahead.  Queries keep their 64 fp16 operand
// registers for the whole loop; K's channels sit in LDS in the order the
// unpack produces them (0, 4, 1, 5, 2, 6, 3, 7 within each group of 8) and the
// query operands use the same order.  Longer key ranges are split over
// several workgroups and folded by the merge kernel.
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
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 4.0f;  // log2 units a score may exceed its row's running max by

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
  // Several sequences in one launch (query rows of a verification round):
  // grid x = sequence * q_tiles + tile; with ctx set, sequence b's T rows sit
  // at positions ctx[b] - T .. ctx[b] - 1 (ctx clamped to [0, max_ctx]; rows
  // at negative positions attend to nothing), its page-table row starts at
  // b * pt_stride and its queries and outputs follow those of sequence b - 1.
  const int32_t* ctx;
  int32_t max_ctx, q_tiles, pt_stride, B;
};

struct __align__(16) PrefillSmem {
  _Float16 k[2][kPage][kKStride];  // K as hi, lo
  _Float16 vt[2][kHeadDim][kPage]; // V^T as hi, lo, tokens in MFMA order, 16-byte chunks swizzled
  uint16_t vsc[2][8][kPage];       // V scales [page parity][block][token]
};

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

typedef _Float16 half2v_t __attribute__((ext_vector_type(2)));

// Exact split of a pair of fp16 scales: hi keeps the top 8 significant bits of
// each, lo = s - hi the rest (at most 3 significant bits).  Both products with
// n - 8 are exact in fp16: they are integer multiples of the scale's last place
// (at least 2^-24, the fp16 subnormal step) with at most 11 and 6 significant
// bits; the matrix cores take fp16 subnormals exactly.
__device__ __forceinline__ void split_scales(uint32_t bits2, half2v_t& hi, half2v_t& lo) {
  hi = __builtin_bit_cast(half2v_t, bits2 & 0xFFF8FFF8u);
  lo = __builtin_bit_cast(half2v_t, bits2) - hi;
}

// Two nibbles at bit offsets sh and 16 + sh of w as the fp16 pair (n0 - 8, n1 - 8).
// magic holds 0x64006400 in a VGPR, so the mask and the OR are one v_and_or_b32
// (an instruction takes one literal constant only).
__device__ __forceinline__ half2v_t nibble_pair(uint32_t w, int sh, uint32_t magic) {
  const uint32_t b = ((w >> sh) & 0x000F000Fu) | magic;  // 1024 + n in each half
  return __builtin_bit_cast(half2v_t, b) + half2v_t{static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
}

__device__ __forceinline__ uint32_t as_u32(half2v_t v) { return __builtin_bit_cast(uint32_t, v); }

// V^T rows.  Within each group of 16 tokens the tokens are stored in the order
// the PV MFMA consumes them, 0-3, 8-11, 4-7, 12-15, so that a lane's 8 operand
// tokens of a k-step are one 16-byte chunk; the row's 8 chunks are
// XOR-permuted by row so that neither the writers of one instruction
// (channel quads, rows 4 apart) nor the readers (consecutive rows) meet on a
// bank.
__device__ __forceinline__ int vt_chunk(int row, int chunk) { return chunk ^ (((row >> 2) ^ (row << 1)) & 7); }

// Cells of one page for this thread, in two parts that are requested at
// different times: the K part (K units (block 2 w + u, token t) for u = 0, 1,
// w = wave, t = lane; the two K scales, adjacent in memory; one dword of the
// page's V scale tile (token tid / 4, blocks 2 (tid % 4), + 1; with one V
// scale per token (VT) tokens 2 (tid % 32), + 1), which goes through LDS) and
// the V part (V units: tokens 8 (2 w + u) .., channel quad j = lane).
struct KRaw {
  uint4 k[2];
  uint32_t ks;   // scales of the two K units, one per half
  uint32_t vsd;  // two V scales of one token
};
struct VRaw {
  uint4 v[2];
};

// Loads of cache cells, with the non-temporal hint (nt: the line is not kept
// for reuse) when NT: in the verification-rows form each (page, KV head) is
// read by one workgroup; the chunk form's pages are read by every query tile
// and stay cacheable.
template <bool NT, typename T>
__device__ __forceinline__ T cell_load(const T* p) {
  if constexpr (NT) {
    if constexpr (sizeof(T) == 16) {
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
      return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
    } else {
      return __builtin_nontemporal_load(p);
    }
  } else {
    return *p;
  }
}

template <bool VT, bool NT>
__device__ __forceinline__ void load_k(const PrefillArgs& a, int64_t ph, int tid, KRaw& r) {
  const uint4* kt = reinterpret_cast<const uint4*>(a.k_nib + ph * (kPage * kHeadDim / 2));
  const uint16_t* ksc = a.k_scale + ph * (kPage * 8);
  const int w = tid >> 6, t = tid & 63;
#pragma unroll
  for (int u = 0; u < 2; ++u) r.k[u] = cell_load<NT>(kt + (2 * w + u) * 64 + t);
  r.ks = cell_load<NT>(reinterpret_cast<const uint32_t*>(ksc + t * 8 + 2 * w));
  if (VT)
    r.vsd = cell_load<NT>(reinterpret_cast<const uint32_t*>(a.v_scale + ph * kPage + 2 * (tid & 31)));
  else
    r.vsd = cell_load<NT>(
        reinterpret_cast<const uint32_t*>(a.v_scale + ph * (kPage * 8) + (tid >> 2) * 8 + 2 * (tid & 3)));
}

template <bool NT>
__device__ __forceinline__ void load_v(const PrefillArgs& a, int64_t ph, int tid, VRaw& r) {
  const uint4* vt = reinterpret_cast<const uint4*>(a.v_nib + ph * (kPage * kHeadDim / 2));
  const int w = tid >> 6, t = tid & 63;
#pragma unroll
  for (int u = 0; u < 2; ++u) r.v[u] = cell_load<NT>(vt + (2 * w + u) * 64 + t);
}

// This thread's dword of the page's V scale tile -> LDS [block][token] (VT:
// row 0 holds the token scales, written by the first 32 threads).
template <bool VT>
__device__ __forceinline__ void store_vscales(PrefillSmem& sm, const KRaw& r, int tid, int parity) {
  if (VT) {
    if (tid < 32) *reinterpret_cast<uint32_t*>(&sm.vsc[parity][0][2 * tid]) = r.vsd;
  } else {
    const int t = tid >> 2, b = 2 * (tid & 3);
    sm.vsc[parity][b][t] = static_cast<uint16_t>(r.vsd);
    sm.vsc[parity][b + 1][t] = static_cast<uint16_t>(r.vsd >> 16);
  }
}

// Dword j of K unit u -> 8 channels of one LDS row [token][channel in unpack
// order], hi and lo.
__device__ __forceinline__ void unpack_k(PrefillSmem& sm, const KRaw& r, int tid, int u, int j, uint32_t magic) {
  const int c = 2 * (tid >> 6) + u, t = tid & 63;
  half2v_t kh, kl;
  split_scales(r.ks, kh, kl);
  const half2v_t s2h{kh[u], kh[u]}, s2l{kl[u], kl[u]};
  const uint32_t w = word(r.k[u], j);
  uint4 hi, lo;
  half2v_t n;
  n = nibble_pair(w, 0, magic);  hi.x = as_u32(n * s2h); lo.x = as_u32(n * s2l);
  n = nibble_pair(w, 4, magic);  hi.y = as_u32(n * s2h); lo.y = as_u32(n * s2l);
  n = nibble_pair(w, 8, magic);  hi.z = as_u32(n * s2h); lo.z = as_u32(n * s2l);
  n = nibble_pair(w, 12, magic); hi.w = as_u32(n * s2h); lo.w = as_u32(n * s2l);
  *reinterpret_cast<uint4*>(&sm.k[0][t][32 * c + 8 * j]) = hi;
  *reinterpret_cast<uint4*>(&sm.k[1][t][32 * c + 8 * j]) = lo;
}

// V unpack, channel 4 j + i of this thread's two V units (tokens 16 g .. 16 g +
// 15, g = wave) -> two 16-byte chunks of V^T row 4 j + i, hi and lo.
// The scales of those 16 tokens come from LDS already paired (tokens 2k, 2k +
// 1), read and split once per page.  The work is cut into 8 pieces of one token pair of
// one unit each: pieces 0-3 fill chunk 2g (tokens 0-3 and 8-11 of the group),
// pieces 4-7 chunk 2g + 1 (tokens 4-7 and 12-15), each chunk written to LDS
// after its fourth piece.
struct VScales {
  half2v_t hi[8], lo[8];  // split scales of tokens 16 g + 2k, + 1 (k = 0..7), block j / 8
};

template <bool VT>
__device__ __forceinline__ void read_vscales(const PrefillSmem& sm, int tid, int parity, VScales& s) {
  const int g = tid >> 6, j = tid & 63;
  const int row = VT ? 0 : j >> 3;  // the lane's block, or the token scales
  const uint4 sa = *reinterpret_cast<const uint4*>(&sm.vsc[parity][row][16 * g]);
  const uint4 sb = *reinterpret_cast<const uint4*>(&sm.vsc[parity][row][16 * g + 8]);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    split_scales(word(sa, k), s.hi[k], s.lo[k]);
    split_scales(word(sb, k), s.hi[4 + k], s.lo[4 + k]);
  }
}

__device__ __forceinline__ void v_piece(PrefillSmem& sm, const VRaw& r, const VScales& s, int tid, int i, int p,
                                        uint32_t* hv, uint32_t* lv, uint32_t magic) {
  const int g = tid >> 6, j = tid & 63;
  const int u = (p >> 1) & 1, k = (p & 1) + 2 * (p >> 2), slot = p & 3;
  const half2v_t n = nibble_pair(word(r.v[u], k), 4 * i, magic);
  hv[slot] = as_u32(n * s.hi[4 * u + k]);
  lv[slot] = as_u32(n * s.lo[4 * u + k]);
  if (slot == 3) {
    const int row = 4 * j + i;
    const int c = vt_chunk(row, 2 * g + (p >> 2));
    *reinterpret_cast<uint4*>(&sm.vt[0][row][8 * c]) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
    *reinterpret_cast<uint4*>(&sm.vt[1][row][8 * c]) = make_uint4(lv[0], lv[1], lv[2], lv[3]);
  }
}

// VT: the cache's V scales are one per token and head.
// ROWS: the query rows of a verification round (at most 8 positions, 32 rows),
// held by every wave: wave w multiplies token tile w & 1 of each page into
// channel half w >> 1 of the output, with its own softmax state over the tokens
// it sees, and the two token tiles of each channel half are folded at the end.
// The page's dequantisation is shared as in the chunk kernel.
template <bool VT, bool ROWS>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a, const int32_t* __restrict__ pt) {
  constexpr int kD = ROWS ? 4 : 8;  // 32-channel tiles of O^T per wave
  __shared__ PrefillSmem sm;
  const int seq = blockIdx.x / a.q_tiles;          // sequence
  const int qt = blockIdx.x - seq * a.q_tiles;     // query tile
  const int g = blockIdx.y;      // KV head
  const int split = blockIdx.z;  // key-range split
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int tt_w = wave & 1, ch_w = wave >> 1;  // ROWS: this wave's token tile and channel half
  int pos0 = a.pos0;
  if (a.ctx) pos0 = min(max(a.ctx[seq], 0), a.max_ctx) - a.T;
  pos0 = __builtin_amdgcn_readfirstlane(pos0);
  pt += static_cast<int64_t>(seq) * a.pt_stride;

  // column tile c of this wave: positions (wave*kCT + c)*8 + col/4, head col % 4
  int qi[kCT], qpos[kCT];
  bool qexists[kCT], qvalid[kCT];
  const int hq = g * kG + (col & 3);
#pragma unroll
  for (int c = 0; c < kCT; ++c) {
    qi[c] = qt * kQPos + ((ROWS ? 0 : wave) * kCT + c) * 8 + col / 4;
    qpos[c] = pos0 + qi[c];
    qexists[c] = qi[c] < a.T;
    qvalid[c] = qexists[c] && qpos[c] >= 0;  // a row at a negative position attends to nothing
  }
  const int qpos_first = pos0 + qt * kQPos;  // no key below it needs a mask

  // key pages this workgroup covers: up to the tile's last position, split evenly
  const int tile_last = pos0 + min(a.T, (qt + 1) * kQPos) - 1;
  const int npages = tile_last < 0 ? 0 : tile_last / kPage + 1;
  const int per = (npages + a.kv_splits - 1) / a.kv_splits;
  // uniform: the division runs on the vector unit, keep the range in scalar registers
  const int pbeg = __builtin_amdgcn_readfirstlane(split * per);
  const int pend = __builtin_amdgcn_readfirstlane(min(npages, pbeg + per));

  // Q^T operands: lane holds q[row][channels of LDS positions 16 s + 8 half + 0..7]
  // for s = 0..15, i.e. channels 8 (2 s + half) + {0, 4, 1, 5, 2, 6, 3, 7}.
  // The wave's query rows are scaled by one power of two 2^qe that brings
  // their largest |q| into [2^10, 2^11) (qe clamped to [-64, 64]), so fp16
  // holds every bf16 query of that range exactly (elements below 2^-27 of the
  // wave's largest round to fp16's subnormal step), and by the sign of the
  // logit scale, so that the scores' maximum is the maximum of the scaled
  // logits.  The wave's logit scale qk = |sm_scale log2(e)| 2^-qe undoes both;
  // a zero logit scale gives zero operands and qk = 1 (every score 0).
  const float qsign = a.qk_scale > 0.0f ? 1.0f : (a.qk_scale < 0.0f ? -1.0f : 0.0f);
  half8_t qf[kCT][16];
  float qk;
  {
    static_assert(kCT == 1, "one query row per lane");
    const uint16_t* qrow =
        a.q + ((static_cast<int64_t>(seq) * a.T + (qexists[0] ? qi[0] : 0)) * a.Hq + hq) * kHeadDim;
    uint4 raw[16];
    float qmax = 0.0f;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      raw[s] = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * half);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = word(raw[s], j);
        qmax = fmaxf(qmax, fmaxf(fabsf(bf16_to_f32(static_cast<uint16_t>(w))),
                                 fabsf(bf16_to_f32(static_cast<uint16_t>(w >> 16)))));
      }
    }
    for (int sh = 32; sh >= 1; sh >>= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, sh, 64));
    int qe = 0;
    if (qmax > 0.0f) {
      int ex;
      frexpf(qmax, &ex);  // qmax in [2^(ex-1), 2^ex)
      qe = min(64, max(-64, 11 - ex));
    }
    qe = __builtin_amdgcn_readfirstlane(qe);
    qk = qsign == 0.0f ? 1.0f : ldexpf(fabsf(a.qk_scale), -qe);
    // wave-uniform: kept in a scalar register, as the plain argument would be
    qk = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, qk)));
#pragma unroll
    for (int s = 0; s < 16; ++s) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = word(raw[s], j);
        const float x0 = qsign * ldexpf(bf16_to_f32(static_cast<uint16_t>(w)), qe);
        const float x1 = qsign * ldexpf(bf16_to_f32(static_cast<uint16_t>(w >> 16)), qe);
        // channels 2j, 2j + 1 of the group go to positions 2j and 2j - 7 (+8 for the odd half)
        qf[0][s][(2 * j) < 4 ? 4 * j : 4 * j - 7] = static_cast<_Float16>(x0);
        qf[0][s][(2 * j + 1) < 4 ? 4 * j + 2 : 4 * j - 5] = static_cast<_Float16>(x1);
      }
    }
  }

  static_assert(kCT == 1, "the page loop below is written for one column tile per wave");
  float16_t acc[kCT][kD];  // O^T per column tile: channel tiles of 32
#pragma unroll
  for (int c = 0; c < kCT; ++c)
#pragma unroll
    for (int d = 0; d < kD; ++d) acc[c][d] = float16_t{};
  float m_run[kCT], s_max[kCT], l_lane[kCT];
#pragma unroll
  for (int c = 0; c < kCT; ++c) {
    m_run[c] = -INFINITY;  // an integer (log2 units) once finite, so rescale factors are powers of two
    s_max[c] = -INFINITY;
    l_lane[c] = 0.0f;
  }

  auto page_handle = [&](int lp, bool& valid) {
    int32_t pid = pt[lp];
    valid = static_cast<uint32_t>(pid) < static_cast<uint32_t>(a.num_pages);
    return static_cast<int64_t>(valid ? pid : 0) * a.Hkv + g;
  };

  // Cells in flight at the top of iteration lp: vcur = V of page lp (unpacked
  // during this page's S work), kraw = K of page lp + 1 (unpacked during this
  // page's PV work); requested now: vnext = V of page lp + 1 and kahead = K of
  // page lp + 2.  The page id of page lp + 3 is read one iteration before its
  // cells are.  Cells past the range are unpacked into buffers nobody reads.
  uint32_t nmagic = 0x64006400u;
  asm volatile("" : "+v"(nmagic));  // kept in a VGPR (see nibble_pair)
  KRaw kraw{}, kahead{};
  VRaw vcur{}, vnext{};
  bool cur_valid = false, kraw_valid = false, kahead_valid = false;
  int64_t kraw_ph = 0, kahead_ph = 0;
  int32_t pid_next = pt[min(pbeg + 2, max(pend - 1, 0))];
  if (pbeg < pend) {
    KRaw k0;
    const int64_t ph0 = page_handle(pbeg, cur_valid);
    load_k<VT, ROWS>(a, ph0, tid, k0);
    load_v<ROWS>(a, ph0, tid, vcur);
    if (pbeg + 1 < pend) {
      kraw_ph = page_handle(pbeg + 1, kraw_valid);
      load_k<VT, ROWS>(a, kraw_ph, tid, kraw);
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) unpack_k(sm, k0, tid, x >> 2, x & 3, nmagic);
    store_vscales<VT>(sm, k0, tid, pbeg & 1);
  }

  // V^T operand addresses of this lane: row col (+ 32 d), chunk (2 (2 tt + s2) + half) swizzled
  const char* vt_lane = reinterpret_cast<const char*>(&sm.vt[0][col][0]);
  int voff[4];
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) voff[c4] = 16 * vt_chunk(col, 2 * c4 + half);

  // ---- the page loop ----------------------------------------------------
  // One wave per SIMD issues everything in order, so the dequantisation and
  // softmax work is cut into small pieces placed between the MFMAs (one piece
  // per MFMA step, each step a scheduling region of its own): the VALU pieces
  // issue while the matrix core works on the step's MFMAs.

  // S^T of one 32-token tile: the K_lo chain, then the K_hi chain into the same
  // accumulator (dependent MFMAs issue back to back).  K operands are read from
  // LDS two steps ahead.
  auto s_phase = [&](int tt, float16_t& st, auto&& piece) {
    auto kread = [&](int step) {
      return *reinterpret_cast<const half8_t*>(&sm.k[step < 16 ? 1 : 0][32 * tt + col][16 * (step & 15) + 8 * half]);
    };
    half8_t kb[3];
    kb[0] = kread(0);
    kb[1] = kread(1);
#pragma unroll
    for (int step = 0; step < 32; ++step) {
      __builtin_amdgcn_sched_barrier(0);
      if (step + 2 < 32) kb[(step + 2) % 3] = kread(step + 2);
      piece(step);
      st = __builtin_amdgcn_mfma_f32_32x32x16_f16(kb[step % 3], qf[0][step & 15], st, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // O^T += V^T P^T for one token tile: step = 8 s2 + d covers k-step s2 (tokens
  // 16 (2 tt + s2) + {0..3, 8..11}, +4 for the upper half lanes) and channel
  // tile d with the MFMAs V_hi P_hi, V_hi P_lo and V_lo P_hi (P_lo V_lo is
  // below fp32 rounding).  V
  // operands are read from LDS a step ahead.
  auto pv_phase = [&](int tt, const half8_t* pb, const half8_t* pl, auto&& piece) {
    auto vread = [&](int step, half8_t* dst) {
      // row d * 32 + col: the swizzle of rows col + 32 d does not depend on d,
      // so the address is a per-lane base plus a constant
      const char* p = vt_lane + voff[tt * 2 + (step >> 3)] + (step & 7) * (32 * kPage * 2);
      dst[0] = *reinterpret_cast<const half8_t*>(p);
      dst[1] = *reinterpret_cast<const half8_t*>(p + kHeadDim * kPage * 2);
    };
    half8_t vbuf[2][2];
    vread(0, vbuf[0]);
#pragma unroll
    for (int step = 0; step < 16; ++step) {
      const int s2 = step >> 3, d = step & 7;
      __builtin_amdgcn_sched_barrier(0);
      if (step + 1 < 16) vread(step + 1, vbuf[(step + 1) & 1]);
      const half8_t* vb = vbuf[step & 1];
      acc[0][d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb[0], pb[s2], acc[0][d], 0, 0, 0);
      acc[0][d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb[0], pl[s2], acc[0][d], 0, 0, 0);
      acc[0][d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb[1], pb[s2], acc[0][d], 0, 0, 0);
      piece(step);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ROWS: O^T += V^T P^T for token tile tt and this wave's 4 channel tiles;
  // step = 4 s2 + d as in pv_phase.
  const char* vt_rows = vt_lane + ch_w * 4 * (32 * kPage * 2);
  int voff_r[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) voff_r[s2] = 16 * vt_chunk(col, 2 * (2 * tt_w + s2) + half);
  auto pv_rows = [&](const half8_t* pb, const half8_t* pl, auto&& piece) {
    auto vread = [&](int step, half8_t* dst) {
      const char* p = vt_rows + voff_r[step >> 2] + (step & 3) * (32 * kPage * 2);
      dst[0] = *reinterpret_cast<const half8_t*>(p);
      dst[1] = *reinterpret_cast<const half8_t*>(p + kHeadDim * kPage * 2);
    };
    half8_t vbuf[2][2];
    vread(0, vbuf[0]);
#pragma unroll
    for (int step = 0; step < 8; ++step) {
      const int s2 = step >> 2, d = step & 3;
      __builtin_amdgcn_sched_barrier(0);
      if (step + 1 < 8) vread(step + 1, vbuf[(step + 1) & 1]);
      const half8_t* vb = vbuf[step & 1];
      acc[0][d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb[0], pb[s2], acc[0][d], 0, 0, 0);
      acc[0][d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb[0], pl[s2], acc[0][d], 0, 0, 0);
      acc[0][d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb[1], pb[s2], acc[0][d], 0, 0, 0);
      piece(step);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Softmax, first part: causal mask where the tile needs it, the row max, and
  // the lazy raise of the running max.  The max moves (and the accumulator and
  // any P operands not yet multiplied are rescaled) only when a score exceeds it
  // by more than kSlack; the new max is rounded up to an integer, so the rescale
  // factor is an exact power of two.  The exact maximum is tracked and restored
  // at the end.  In pieces, for the matrix phases: part 0 masks the tile where
  // needed and takes the maximum of its first 8 scores, part 1 that of the
  // other 8 and starts the exchange with the other half's row, max_finish
  // settles the row maximum and the lazy raise.
  auto max_part = [&](float16_t& st, int lp, int tt, int part, float& mx, float& other) {
    if (part == 0) {
      const bool need_mask = !cur_valid || lp * kPage + tt * 32 + 31 > qpos_first;
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tok = lp * kPage + tt * 32 + (i / 4) * 8 + half * 4 + (i % 4);
          const bool ok = cur_valid && qvalid[0] && tok <= qpos[0];
          st[i] = ok ? st[i] : -INFINITY;
        }
      }
      mx = st[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, st[i]);
    } else {
#pragma unroll
      for (int i = 8; i < 16; ++i) mx = fmaxf(mx, st[i]);
      other = __shfl_xor(mx, 32, 64);
    }
  };
  auto max_finish = [&](float mx, float other, half8_t* pb_prev, half8_t* pl_prev) {
    mx = fmaxf(mx, other) * qk;  // log2 units
    s_max[0] = fmaxf(s_max[0], mx);
    const bool raise = mx > m_run[0] + kSlack;
    if (__ballot(raise)) {
      const float mn = raise ? ceilf(mx) : m_run[0];
      const float alpha = m_run[0] == -INFINITY ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, static_cast<int>(m_run[0] - mn));
      m_run[0] = mn;
      l_lane[0] *= alpha;
#pragma unroll
      for (int d = 0; d < kD; ++d) acc[0][d] *= alpha;
      if (pb_prev) {
        const _Float16 ah = static_cast<_Float16>(alpha);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          pb_prev[s2] *= ah;
          pl_prev[s2] *= ah;
        }
      }
    }
  };

  // The whole first part at once (the ROWS form).
  auto softmax_max = [&](float16_t& st, int lp, int tt) {
    float mx, other;
    max_part(st, lp, tt, 0, mx, other);
    max_part(st, lp, tt, 1, mx, other);
    max_finish(mx, other, nullptr, nullptr);
  };

  // Softmax, second part, in half-pieces of one score pair (2j, 2j + 1): the
  // even half exponentiates, the odd half splits.  B operands per k-step: P *
  // 2^11 as hi and lo (rounded toward zero).  P stays below 2^kSlack, so P *
  // 2^11 fits fp16; the power-of-two offset keeps all but negligible weights
  // out of the subnormal range.  The accumulator carries P * 2^11 throughout
  // and the epilogue divides it out.
  auto p_half = [&](const float16_t& st, float off, int h, float* e, float& psum, half8_t* pb, half8_t* pl) {
    const int j = h >> 1;
    if ((h & 1) == 0) {
      e[0] = __builtin_amdgcn_exp2f(fmaf(st[2 * j], qk, off));
      e[1] = __builtin_amdgcn_exp2f(fmaf(st[2 * j + 1], qk, off));
    } else {
      psum += e[0] + e[1];
      const auto hh = __builtin_amdgcn_cvt_pkrtz(e[0], e[1]);
      // e - hi as one mixed-precision FMA each (fp16 operand from the packed pair)
      const uint32_t hb = __builtin_bit_cast(uint32_t, hh);
      float d0, d1;
      asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d0) : "v"(hb), "v"(e[0]));
      asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d1) : "v"(hb), "v"(e[1]));
      const auto ll = __builtin_amdgcn_cvt_pkrtz(d0, d1);
      pb[j / 4][2 * (j % 4)] = static_cast<_Float16>(hh[0]);
      pb[j / 4][2 * (j % 4) + 1] = static_cast<_Float16>(hh[1]);
      pl[j / 4][2 * (j % 4)] = static_cast<_Float16>(ll[0]);
      pl[j / 4][2 * (j % 4) + 1] = static_cast<_Float16>(ll[1]);
    }
  };
  auto p_offset = [&]() { return 11.0f - (m_run[0] == -INFINITY ? 0.0f : m_run[0]); };

  for (int lp = pbeg; lp < pend; ++lp) {
    // read before this iteration's cell loads, so that waiting for it next
    // iteration does not wait for them (a clamped index keeps the read in range)
    const int32_t pid_after = pt[min(lp + 3, pend - 1)];
    if (lp + 2 < pend) {
      kahead_valid = static_cast<uint32_t>(pid_next) < static_cast<uint32_t>(a.num_pages);
      kahead_ph = static_cast<int64_t>(kahead_valid ? pid_next : 0) * a.Hkv + g;
      load_k<VT, ROWS>(a, kahead_ph, tid, kahead);
    }
    if (lp + 1 < pend) load_v<ROWS>(a, kraw_ph, tid, vnext);
    pid_next = pid_after;
    __syncthreads();  // K of this page is in LDS; every wave is done with the previous V
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (ROWS) {
      // ---- S^T of this wave's token tile, this thread's V units unpacked meanwhile ----
      VScales vs;
      read_vscales<VT>(sm, tid, lp & 1, vs);
      uint32_t hv[4], lv[4];
      float16_t st{};
      s_phase(tt_w, st, [&](int step) { v_piece(sm, vcur, vs, tid, step >> 3, step & 7, hv, lv, nmagic); });
      softmax_max(st, lp, tt_w);
      half8_t pb[2], pl[2];
      float e[2], psum = 0.0f;
      const float off = p_offset();
#pragma unroll
      for (int h = 0; h < 16; ++h) p_half(st, off, h, e, psum, pb, pl);
      l_lane[0] += psum * (1.0f / 2048.0f);
      __syncthreads();  // V of this page is in LDS; every wave is done with this K
      __builtin_amdgcn_sched_barrier(0);

      // ---- PV of this wave's tile and channel half, the next page's K meanwhile ----
      pv_rows(pb, pl, [&](int step) {
        unpack_k(sm, kraw, tid, step >> 2, step & 3, nmagic);
        if (step == 7) store_vscales<VT>(sm, kraw, tid, (lp + 1) & 1);
      });
    } else {
    // ---- tile 0: S^T, V channels 0-2 of this page unpacked meanwhile ----
    VScales vs;
    read_vscales<VT>(sm, tid, lp & 1, vs);
    uint32_t hv[4], lv[4];
    float16_t st0{};
    s_phase(0, st0, [&](int step) {
      if (step < 24) v_piece(sm, vcur, vs, tid, step >> 3, step & 7, hv, lv, nmagic);
    });

    // ---- tile 1: S^T; tile 0's maximum (in pieces), the last V channel and tile 0's P meanwhile ----
    half8_t pb0[2], pl0[2], pb1[2], pl1[2];
    float e[2], psum = 0.0f;
    float off0 = 0.0f, mx0 = 0.0f, ot0 = 0.0f;
    float16_t st1{};
    s_phase(1, st1, [&](int step) {
      if (step == 1 || step == 2) {
        max_part(st0, lp, 0, step - 1, mx0, ot0);
      } else if (step == 5) {
        max_finish(mx0, ot0, nullptr, nullptr);
        off0 = p_offset();
      } else if (step >= 6 && step < 30) {  // (steps 3 and 4: the exchange of the row maximum is in flight)
        if (step < 14)
          v_piece(sm, vcur, vs, tid, 3, step - 6, hv, lv, nmagic);
        else
          p_half(st0, off0, step - 14, e, psum, pb0, pl0);
      }
    });
    l_lane[0] += psum * (1.0f / 2048.0f);
    // keeps tile 0's P inside that phase (it would otherwise sink to its first use)
    asm volatile("" ::"v"(pb0[0]), "v"(pb0[1]), "v"(pl0[0]), "v"(pl0[1]));
    __syncthreads();  // V of this page is in LDS; every wave is done with this K
    __builtin_amdgcn_sched_barrier(0);

    // ---- PV of tile 0; tile 1's maximum (in pieces), its P and K channels of the next page meanwhile ----
    // A raise of the maximum here rescales the accumulator (with the products
    // of tile 0 already in it) and the P operands of tile 0 not yet
    // multiplied, by the same power of two.
    float off1 = 0.0f, mx1 = 0.0f, ot1 = 0.0f;
    psum = 0.0f;
    pv_phase(0, pb0, pl0, [&](int step) {
      if (step == 0 || step == 1) {
        max_part(st1, lp, 1, step, mx1, ot1);
      } else if (step == 3) {
        max_finish(mx1, ot1, pb0, pl0);
        off1 = p_offset();
      } else if (step >= 4 && step < 12) {
        p_half(st1, off1, 2 * (step - 4), e, psum, pb1, pl1);
        p_half(st1, off1, 2 * (step - 4) + 1, e, psum, pb1, pl1);
      } else if (step >= 12) {
        unpack_k(sm, kraw, tid, (step - 12) >> 2, (step - 12) & 3, nmagic);
      }
    });
    l_lane[0] += psum * (1.0f / 2048.0f);
    asm volatile("" ::"v"(pb1[0]), "v"(pb1[1]), "v"(pl1[0]), "v"(pl1[1]));

    // ---- PV of tile 1, the rest of the next page's K meanwhile ----
    pv_phase(1, pb1, pl1, [&](int step) {
      if (step < 4)
        unpack_k(sm, kraw, tid, (step + 4) >> 2, (step + 4) & 3, nmagic);
      else if (step == 4)
        store_vscales<VT>(sm, kraw, tid, (lp + 1) & 1);
    });
    }

    vcur = vnext;
    cur_valid = kraw_valid;
    kraw = kahead;
    kraw_ph = kahead_ph;
    kraw_valid = kahead_valid;
  }


  if constexpr (ROWS) {
    // Fold the two token tiles of each channel half: the tile-1 wave leaves its
    // state in LDS (lane-contiguous rows of floats), the tile-0 wave adds it.
    // Both running maxima are integers, so the factors are exact powers of two.
    __syncthreads();  // every wave is done with the page tiles
    constexpr int kX = kD * 16 + 3;
    float* xs = reinterpret_cast<float*>(&sm.k[0][0][0]) + ch_w * kX * 64;
    static_assert(2 * kX * 64 * sizeof(float) <= sizeof(sm.k), "fold buffer fits the K tiles");
    if (tt_w == 1) {
#pragma unroll
      for (int d = 0; d < kD; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) xs[(d * 16 + i) * 64 + lane] = acc[0][d][i];
      xs[(kD * 16) * 64 + lane] = m_run[0];
      xs[(kD * 16 + 1) * 64 + lane] = s_max[0];
      xs[(kD * 16 + 2) * 64 + lane] = l_lane[0];
    }
    __syncthreads();
    if (tt_w == 1) return;
    const float m1 = xs[(kD * 16) * 64 + lane], s1 = xs[(kD * 16 + 1) * 64 + lane];
    const float l1 = xs[(kD * 16 + 2) * 64 + lane];
    const float M = fmaxf(m_run[0], m1);
    const float a0 = m_run[0] == -INFINITY ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, static_cast<int>(m_run[0] - M));
    const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, static_cast<int>(m1 - M));
#pragma unroll
    for (int d = 0; d < kD; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[0][d][i] = acc[0][d][i] * a0 + xs[(d * 16 + i) * 64 + lane] * a1;
    l_lane[0] = l_lane[0] * a0 + l1 * a1;
    s_max[0] = fmaxf(s_max[0], s1);
    m_run[0] = M;
  }

  // ---- epilogue: this lane's query row (ROWS: this wave's channel half) ----
  const int64_t R = static_cast<int64_t>(a.B) * a.T * a.Hq;
  const int d0 = ROWS ? 4 * ch_w : 0;  // first channel tile of acc
#pragma unroll
  for (int c = 0; c < kCT; ++c) {
    // restore the exact maximum: the normalised output is unchanged, the sum scales
    const float f = s_max[c] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[c] - s_max[c]);
    const float Lr = l_lane[c] + __shfl_xor(l_lane[c], 32, 64);  // in units of exp2(m_run)
    const float L = Lr * f;
    if (!qexists[c]) continue;
    const int64_t row = split * R + (static_cast<int64_t>(seq) * a.T + qi[c]) * a.Hq + hq;
    const float inv = Lr > 0.0f ? 1.0f / (Lr * 2048.0f) : 0.0f;  // P was carried times 2^11
    float* dst = a.o + row * kHeadDim;
#pragma unroll
    for (int d = 0; d < kD; ++d)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float4_t v;
        v.x = acc[c][d][4 * i4 + 0] * inv;
        v.y = acc[c][d][4 * i4 + 1] * inv;
        v.z = acc[c][d][4 * i4 + 2] * inv;
        v.w = acc[c][d][4 * i4 + 3] * inv;
        *reinterpret_cast<float4_t*>(dst + (d0 + d) * 32 + i4 * 8 + half * 4) = v;
      }
    if (half == 0 && (!ROWS || wave == 0)) {
      if (a.m) a.m[row] = L > 0.0f ? s_max[c] * kLn2 : -INFINITY;
      if (a.l) a.l[row] = L;
    }
  }
}

}  // namespace

PrefillPlan plan_prefill(int32_t T, int32_t Hq, int32_t Hkv, int32_t pos0, int32_t tile_positions,
                         int32_t target_wgs) {
  PrefillPlan p;
  p.q_tiles = (T + tile_positions - 1) / tile_positions;
  const int64_t total_pages = (static_cast<int64_t>(pos0) + T + kPage - 1) / kPage;
  // split the key range until the grid reaches the target when the range is
  // long (a short chunk over a long window gets as many splits as it needs to
  // fill the device), keeping at least 16 pages per split
  // (rounded down: a grid just past a whole number of rounds would add a
  // round of a few workgroups that takes as long as a full one)
  const int64_t wgs = static_cast<int64_t>(p.q_tiles) * Hkv;
  int64_t splits = target_wgs / std::max<int64_t>(wgs, 1);
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, total_pages / 16));
  p.kv_splits = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(splits, 1024)));
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
  a.ctx = nullptr;
  a.max_ctx = 0;
  a.q_tiles = plan.q_tiles;
  a.pt_stride = 0;
  a.B = 1;
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
  if (c.v_scale_per_token)
    hipLaunchKernelGGL((prefill_kernel<true, false>), dim3(plan.q_tiles, a.Hkv, plan.kv_splits), dim3(kThreads), 0, s, a, pt);
  else
    hipLaunchKernelGGL((prefill_kernel<false, false>), dim3(plan.q_tiles, a.Hkv, plan.kv_splits), dim3(kThreads), 0, s, a,
                       pt);
  hipError_t e = hipGetLastError();
  timing_end(F4KV_KERNEL_PREFILL, s);
  if (e != hipSuccess || plan.kv_splits == 1) return e;
  return launch_merge(pm, pl, a.o, plan.kv_splits, static_cast<int32_t>(R), kHeadDim, out, out_m, out_l, s);
}

// Five or more rows of a group of 4 query heads (20 or more rows per KV head,
// three or more passes of the decode kernel over the pages) go through this
// kernel, whose workgroup reads each page once for up to 32 rows with
// matrix-core products (the ROWS form: the four waves share the rows and
// split each page's tokens and output channels): a verification round is a
// short causal prefill over the cache.  Whole-context calls only.
int32_t rows_prefill_splits(int32_t B, int32_t R, int32_t Hq, int32_t Hkv, int32_t max_ctx, int32_t num_windows,
                            int32_t window_tokens) {
  if (R < 5 || R > 8 || Hq != 4 * Hkv || num_windows != 1 || window_tokens != 0 || B <= 0) return 0;
  const int64_t wgs = static_cast<int64_t>(B) * Hkv;
  const int64_t total_pages = (static_cast<int64_t>(max_ctx) + kPage - 1) / kPage;
  int64_t splits = 512 / wgs;  // at most two rounds of one workgroup per CU, as the prefill plans
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, total_pages / 16));
  return static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(splits, 1024)));
}

size_t rows_prefill_ws_bytes(int32_t B, int32_t R, int32_t Hq, int32_t splits) {
  const int64_t rows = static_cast<int64_t>(B) * R * Hq;
  return splits > 1 ? static_cast<size_t>(splits) * rows * (kHeadDim + 2) * sizeof(float) : 0;
}

// R <= 8 query rows of each of B sequences, row r at position ctx[b] - R + r,
// causal over the cache: one query tile per sequence (every wave holds its
// rows), the key range split kv_splits ways and folded by the merge.
hipError_t launch_prefill_rows(const f4kv_cache& c, const uint16_t* q, const int32_t* pt, const int32_t* ctx,
                               int32_t B, int32_t R, int32_t Hq, int32_t max_pages, int32_t max_ctx, float sm_scale,
                               float* out, float* out_m, float* out_l, void* ws, int32_t kv_splits, hipStream_t s) {
  if (B == 0) return hipSuccess;
  PrefillArgs a;
  a.k_nib = c.k_nib;
  a.k_scale = c.k_scale;
  a.v_nib = c.v_nib;
  a.v_scale = c.v_scale;
  a.q = q;
  a.pt = pt;
  a.T = R;
  a.Hq = Hq;
  a.Hkv = c.num_kv_heads;
  a.num_pages = c.num_pages;
  a.max_pages = max_pages;
  a.pos0 = 0;
  a.kv_splits = kv_splits;
  a.qk_scale = sm_scale * kLog2e;
  a.ctx = ctx;
  a.max_ctx = max_ctx;
  a.q_tiles = 1;
  a.pt_stride = max_pages;
  a.B = B;
  const int64_t rows = static_cast<int64_t>(B) * R * Hq;
  float* pm = nullptr;
  float* pl = nullptr;
  if (kv_splits > 1) {
    float* base = static_cast<float*>(ws);
    a.o = base;
    pm = base + static_cast<size_t>(kv_splits) * rows * kHeadDim;
    pl = pm + static_cast<size_t>(kv_splits) * rows;
    a.m = pm;
    a.l = pl;
  } else {
    a.o = out;
    a.m = out_m;
    a.l = out_l;
  }
  const dim3 grid(B, a.Hkv, kv_splits);
  timing_begin(F4KV_KERNEL_PREFILL, s);
  if (c.v_scale_per_token)
    hipLaunchKernelGGL((prefill_kernel<true, true>), grid, dim3(kThreads), 0, s, a, pt);
  else
    hipLaunchKernelGGL((prefill_kernel<false, true>), grid, dim3(kThreads), 0, s, a, pt);
  hipError_t e = hipGetLastError();
  timing_end(F4KV_KERNEL_PREFILL, s);
  if (e != hipSuccess || kv_splits == 1) return e;
  return launch_merge(pm, pl, a.o, kv_splits, static_cast<int32_t>(rows), kHeadDim, out, out_m, out_l, s);
}

}  // namespace f4kv
