// Device routines shared by several kernels, so that a fused launch computes
// bit for bit what the separate entry points compute: the NEOX rotation of one
// channel pair (yarn_rope_apply) and the F4 block quantiser and cell stores
// (kv_cache_write_f4).
#pragma once

#include "f4kv_internal.h"

namespace f4kv {

// Rotation of the pair (x0, x1) = (x[e], x[e + rotary_dim / 2]) by the angle
// whose cosine and sine rows hold c and s (the NEOX rotation with the
// statically YaRN-scaled table: mistral.rs PR #2375, "Changes by area" item 1),
// in fp64 with the two fused multiply-adds written out, so every caller rounds
// the same way.
__device__ __forceinline__ void rope_rotate_pair(double x0, double x1, double c, double s, double& y0,
                                                 double& y1) {
  y0 = __builtin_fma(x0, c, -(x1 * s));
  y1 = __builtin_fma(x1, c, x0 * s);
}

// One 32-value block to F4 (mistral.rs PR #2375, "Changes by area" item 2:
// (nibble - 8) * scale): scale = fp16(amax / 8) (nearest even, saturated at
// 65504; amax * 0.125 is exact in fp32, so one rounding), code = rne(x / s)
// clamped to [-8, 7], nibble = code + 8.  The quotient is formed in fp64: an
// inexact fp32 x / fp16 s lies at least 2^-24 |x / s| from any half-integer,
// so fp64 decides every tie and near-tie exactly.  amax is the block's
// absolute maximum, or the row's when V carries one scale per token.
// Returns the scale's fp16 bits.
// The block's scale: its fp16 bits, and its value in fp64 for the quotients.
__device__ __forceinline__ uint16_t f4_scale(float amax, double& sd) {
  const _Float16 s16 = static_cast<_Float16>(fminf(amax * 0.125f, 65504.0f));
  sd = static_cast<double>(static_cast<float>(s16));
  return __builtin_bit_cast(uint16_t, s16);
}

// The nibble of one value under the scale sd (0 codes to 8 when sd is 0).
__device__ __forceinline__ uint32_t f4_nibble(float x, double sd) {
  int code = 0;
  if (sd > 0.0) {
    double qd = __builtin_rint(static_cast<double>(x) / sd);
    qd = fmin(fmax(qd, -8.0), 7.0);
    code = static_cast<int>(qd);
  }
  return static_cast<uint32_t>(code + 8);
}

__device__ __forceinline__ uint16_t f4_quantize_block(const float* x, float amax, uint32_t* nib) {
  double sd;
  const uint16_t sbits = f4_scale(amax, sd);
#pragma unroll
  for (int i = 0; i < kBlock; ++i) nib[i] = f4_nibble(x[i], sd);
  return sbits;
}

// K block c of token slot `off` in page-head ph (= page * H + head): 16 bytes
// in the block-major K tile [D/32][64][16] and its scale [64][D/32].
__device__ __forceinline__ void f4_store_k_block(uint8_t* k_nib, uint16_t* k_scale, int64_t ph, int nb, int c,
                                                 int off, const uint32_t* nib, uint16_t sbits) {
  uint32_t w[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t v = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) v |= nib[8 * d + e] << (4 * e);
    w[d] = v;
  }
  uint8_t* dst = k_nib + ((ph * nb + c) * kPage + off) * 16;
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  k_scale[(ph * kPage + off) * nb + c] = sbits;
}

// V block c of token slot `off` in page-head ph: the V tile [8][D/4][16] keeps
// 8 tokens x 4 channels per 16-byte unit, two tokens per dword, so the block's
// 8 channel quads go to 8 units as 2-byte pieces; the scale goes to [64][D/32],
// or (one scale per token) to [64], written by the thread of block 0.
__device__ __forceinline__ void f4_store_v_block(uint8_t* v_nib, uint16_t* v_scale, int64_t ph, int D, int c,
                                                 int off, const uint32_t* nib, uint16_t sbits, bool per_token) {
  const int nb = D / kBlock;
  const int quads = D / 4;
  uint8_t* tile = v_nib + ph * (static_cast<int64_t>(kPage) * D / 2);
  const int unit_c = off / 8;
  const int byte_in_unit = 4 * ((off % 8) / 2) + 2 * (off % 2);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int j = c * 8 + q;  // dim quad 4j .. 4j+3
    const uint32_t b0 = nib[4 * q + 0] | (nib[4 * q + 1] << 4);
    const uint32_t b1 = nib[4 * q + 2] | (nib[4 * q + 3] << 4);
    uint16_t* dst = reinterpret_cast<uint16_t*>(tile + (static_cast<int64_t>(unit_c) * quads + j) * 16 + byte_in_unit);
    *dst = static_cast<uint16_t>(b0 | (b1 << 8));
  }
  if (!per_token)
    v_scale[(ph * kPage + off) * nb + c] = sbits;
  else if (c == 0)
    v_scale[ph * kPage + off] = sbits;
}

}  // namespace f4kv
