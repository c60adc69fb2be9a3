// Internal declarations shared by the library's translation units (HIP path only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "f4kv.h"

namespace f4kv {

constexpr int kPage = 64;      // tokens per page
constexpr int kBlock = 32;     // values per scale block
constexpr int kHeadDim = 256;  // head_dim the attention kernels implement

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- scalar conversions (device) --------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, nearest-even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float f16bits_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ uint16_t f32_to_f16bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// ---- kernel timing (host) ----------------------------------------------------
// Record the start / end event of one timed launch of `kernel` on stream s
// (no-ops unless f4kv_timing_start is active for that kernel).
void timing_begin(int kernel, hipStream_t s);
void timing_end(int kernel, hipStream_t s);
hipError_t timing_start(int kernel, int max_launches);
hipError_t timing_stop(int kernel, double* total_ms, int64_t* launches);

// ---- device-side checks (host); see f4kv_device_checks ----------------------
bool checks_on();
void set_checks(bool on);
hipError_t read_check_word(uint32_t* out);
// context lengths (or one fixed length when ctx is null) and the page ids of
// the live pages of B page-table rows
hipError_t check_pages(const int32_t* ctx, int32_t fixed_len, const int32_t* pt, int32_t B, int32_t max_pages,
                       int32_t max_ctx, int32_t num_pages, hipStream_t s);
hipError_t check_slots(const int32_t* slots, int32_t T, int64_t num_slots, hipStream_t s);
hipError_t check_rows(const int32_t* cu, int32_t B, const int32_t* pt, int32_t max_pages, int32_t total,
                      int32_t num_pages, hipStream_t s);

// ---- kernel launchers (host); arguments already validated ------------------
hipError_t launch_kv_write(const f4kv_cache& c, const float* k, const float* v,
                           const int32_t* slots, int32_t T, hipStream_t s);

// Same, with slot = page_table[(pos0 + t) / 64] * 64 + (pos0 + t) % 64.
hipError_t launch_kv_write_paged(const f4kv_cache& c, const float* k, const float* v,
                                 const int32_t* page_table, int32_t pos0, int32_t T, hipStream_t s);

hipError_t launch_rope_table(const f4kv_yarn_params& p, double mscale, const int32_t* pos,
                             int32_t n, float* cos_out, float* sin_out, hipStream_t s);

hipError_t launch_rope_apply(const float* c, const float* sn, const void* x, int32_t xdt,
                             void* y, int32_t ydt, int32_t T, int32_t H, int32_t D,
                             int32_t rd, hipStream_t s);

hipError_t launch_merge(const float* m, const float* l, const float* o, int32_t C, int32_t R,
                        int32_t D, float* out, float* out_m, float* out_l, hipStream_t s);

hipError_t launch_gather(const f4kv_cache& c, const int32_t* pt, const int32_t* cu, int32_t B, int32_t max_pages,
                         int32_t total, void* k_out, void* v_out, bool bf16, hipStream_t s);

struct DecodePlan {
  int32_t per_head_target;   // work items per KV head that fill the GPU once
  int32_t max_items;         // bound on the work items of any context lengths
  size_t part_o_offset, part_ml_offset, items_offset, count_offset, qprep_offset;
  size_t ws_bytes;           // workspace the call needs
};

// R query rows per sequence (row r at position ctx - R + r); R == 1 is plain decode.
DecodePlan plan_decode(int32_t B, int32_t R, int32_t Hq, int32_t Hkv, int32_t max_ctx,
                       int32_t num_windows, int32_t window_tokens);

// Fixed device-side workspace for the allocation-free decode entry point: its
// size, and its device address on the current device (looked up on first use).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** ptr);

// The new token of each sequence, for a decode step that rotates the queries
// and rotates and writes the token's K and V before attending (R == 1):
// cos / sin [B][rotary_dim / 2], k_new / v_new fp32 [B][Hkv][D], slots [B].
struct DecodeStep {
  const float* cos;
  const float* sin;
  int32_t rotary_dim;
  const float* k_new;
  const float* v_new;
  const int32_t* slots;
};

// step: null for a plain decode (q already rotated).
hipError_t launch_decode(const f4kv_cache& c, const uint16_t* q, const int32_t* pt,
                         const int32_t* ctx, int32_t B, int32_t R, int32_t Hq, int32_t max_pages,
                         int32_t max_ctx, int32_t num_windows, int32_t window_tokens,
                         float sm_scale, float* out, float* out_m, float* out_l,
                         void* ws, const DecodePlan& plan, const DecodeStep* step, hipStream_t s);

// Query rows of B sequences (row r at position ctx[b] - R + r) through the
// prefill kernel: 4 query heads per KV head, head_dim 256, R <= 8.
// rows_prefill_splits gives the key splits of such a launch, or 0 when the
// call stays on the decode kernel; rows_prefill_ws_bytes its workspace.
int32_t rows_prefill_splits(int32_t B, int32_t R, int32_t Hq, int32_t Hkv, int32_t max_ctx, int32_t num_windows,
                            int32_t window_tokens);
size_t rows_prefill_ws_bytes(int32_t B, int32_t R, int32_t Hq, int32_t splits);
hipError_t launch_prefill_rows(const f4kv_cache& c, const uint16_t* q, const int32_t* pt, const int32_t* ctx,
                               int32_t B, int32_t R, int32_t Hq, int32_t max_pages, int32_t max_ctx, float sm_scale,
                               float* out, float* out_m, float* out_l, void* ws, int32_t kv_splits, hipStream_t s);

struct PrefillPlan {
  int32_t q_tiles;      // query tiles of 32 positions
  int32_t kv_splits;    // workgroups along the key range per query tile
  size_t ws_bytes;
};

// tile_positions query positions per workgroup; the key range is split until
// the grid has about target_wgs workgroups (at most 1024 splits, each >= 16 pages).
PrefillPlan plan_prefill(int32_t T, int32_t Hq, int32_t Hkv, int32_t pos0, int32_t tile_positions,
                         int32_t target_wgs);
// The plans of the two prefill kernels (fp16: 32 positions, two workgroup
// rounds; 8-bit: 64 positions, one round).
inline PrefillPlan plan_prefill_f16(int32_t T, int32_t Hq, int32_t Hkv, int32_t pos0) {
  return plan_prefill(T, Hq, Hkv, pos0, 32, 512);
}
inline PrefillPlan plan_prefill_fp8(int32_t T, int32_t Hq, int32_t Hkv, int32_t pos0) {
  return plan_prefill(T, Hq, Hkv, pos0, 64, 256);
}

hipError_t launch_prefill(const f4kv_cache& c, const uint16_t* q, const int32_t* pt,
                          int32_t max_pages, int32_t T, int32_t Hq, int32_t pos0,
                          float sm_scale, float* out, float* out_m, float* out_l,
                          void* ws, const PrefillPlan& plan, hipStream_t s);

// The same chunk with 8-bit products (Q.K^T in INT8, P.V in E4M3); same plan.
hipError_t launch_prefill_fp8(const f4kv_cache& c, const uint16_t* q, const int32_t* pt,
                              int32_t max_pages, int32_t T, int32_t Hq, int32_t pos0,
                              float sm_scale, float* out, float* out_m, float* out_l,
                              void* ws, const PrefillPlan& plan, hipStream_t s);

}  // namespace f4kv
