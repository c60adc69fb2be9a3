// Measured ceilings of the GPU the benchmark runs on: a plain HBM read kernel,
// the decode kernel's paged loads without its arithmetic, and matrix-core loops (fp16, E4M3 and INT8 products, the instructions the
// prefill kernels issue).  bench.py reports the library's rates against these
// beside the nominal peaks.  Not part of the library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A 16-byte load, with the non-temporal hint (nt: the line is not kept for
// reuse) when NT.
template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

// Every thread streams 16-byte words with a grid-stride loop, U loads in
// flight per iteration; the XOR of all words is kept so that no load can be
// dropped (it is written out only if it hits a value the data never makes).
template <int U, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = ld<NT>(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = ld<NT>(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// The loads of the decode kernel without its arithmetic: for B sequences of
// n_pages pages and Hkv KV heads, per (page, head) the K tile (8 KB), its
// scale row (1 KB), then the V tile (8 KB) and its scale row (1 KB), 16-byte
// loads with lane = 16-byte column as in the decode kernel.  Work split as in
// the decode kernel: a workgroup of 4 waves owns a contiguous range of one
// (sequence, head)'s pages, wave w takes every 4th page of it.
template <bool NT>
__global__ __launch_bounds__(256) void paged_read_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                                         const u32x4* __restrict__ ks,
                                                         const u32x4* __restrict__ vs, const int32_t* __restrict__ pt,
                                                         int B, int max_pages, int n_pages, int Hkv,
                                                         int chunks_per_head, uint32_t* __restrict__ sink) {
  const int x = blockIdx.x;
  const int bh = x / chunks_per_head, c = x % chunks_per_head;
  if (bh >= B * Hkv) return;
  const int b = bh / Hkv, h = bh % Hkv;
  const int per = (n_pages + chunks_per_head - 1) / chunks_per_head;
  const int p0 = c * per, p1 = min(n_pages, p0 + per);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint32_t acc = 0;
  for (int p = p0 + wave; p < p1; p += 4) {
    const int64_t ph = static_cast<int64_t>(pt[static_cast<int64_t>(b) * max_pages + p]) * Hkv + h;
    u32x4 w[9];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = ld<NT>(k + ph * 512 + i * 64 + lane);  // 512 x 16 B per tile
    w[8] = ld<NT>(ks + ph * 64 + lane);                                        // 64 x 16 B per scale row
#pragma unroll
    for (int i = 0; i < 9; ++i) acc ^= w[i].x ^ w[i].y ^ w[i].z ^ w[i].w;
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = ld<NT>(v + ph * 512 + i * 64 + lane);
    w[8] = ld<NT>(vs + ph * 64 + lane);
#pragma unroll
    for (int i = 0; i < 9; ++i) acc ^= w[i].x ^ w[i].y ^ w[i].z ^ w[i].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Four independent accumulator chains per wave, `iters` rounds.  The operands
// come from the thread index so nothing folds; the accumulators are written
// only under a condition the caller never meets (iters < 0 is refused).
template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ sink) {
  const int t = threadIdx.x;
  if (KIND == 0) {
    half8_t a, b;
    for (int j = 0; j < 8; ++j) {
      a[j] = static_cast<_Float16>((t + j) & 7);
      b[j] = static_cast<_Float16>((t * 3 + j) & 7);
    }
    f32x16 c0{}, c1{}, c2{}, c3{};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, b, c3, 0, 0, 0);
    }
    if (c0[0] + c1[1] + c2[2] + c3[3] == -1.0f) sink[t] = c0[5];
  } else if (KIND == 1) {
    i32x8 a, b;
    for (int j = 0; j < 8; ++j) {
      a[j] = 0x38383838 + ((t + j) & 3);  // E4M3 values near 1
      b[j] = 0x30303030 + ((t * 3 + j) & 3);
    }
    f32x16 c0{}, c1{}, c2{}, c3{};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 0, 0, 0, 127, 0, 127);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 0, 0, 0, 127, 0, 127);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 0, 0, 0, 127, 0, 127);
    }
    if (c0[0] + c1[1] + c2[2] + c3[3] == -1.0f) sink[t] = c0[5];
  } else {
    i32x4 a, b;
    for (int j = 0; j < 4; ++j) {
      a[j] = 0x01010101 * ((t + j) & 7);
      b[j] = 0x01010101 * ((t * 3 + j) & 7);
    }
    i32x16 c0{}, c1{}, c2{}, c3{};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    if (c0[0] + c1[1] + c2[2] + c3[3] == -1) sink[t] = static_cast<float>(c0[5]);
  }
}

template <int U>
void launch_stream_read(const u32x4* p, size_t n, uint32_t* sink, int grid, bool nt, hipStream_t stream) {
  if (nt)
    hipLaunchKernelGGL(HIP_KERNEL_NAME(stream_read_kernel<U, true>), dim3(grid), dim3(256), 0, stream, p, n, sink);
  else
    hipLaunchKernelGGL(HIP_KERNEL_NAME(stream_read_kernel<U, false>), dim3(grid), dim3(256), 0, stream, p, n, sink);
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) at buf with `grid` workgroups of 256
// threads on `stream`, `unroll` (4, 8 or 16) loads in flight per thread, with
// the non-temporal hint when nt != 0.  sink: one device word.  0 = launched.
int ceiling_stream_read(const void* buf, size_t bytes, uint32_t* sink, int grid, int unroll, int nt,
                        hipStream_t stream) {
  if (!buf || !sink || bytes % 16 != 0 || grid <= 0) return 1;
  const u32x4* p = static_cast<const u32x4*>(buf);
  const size_t n = bytes / 16;
  if (unroll == 4)
    launch_stream_read<4>(p, n, sink, grid, nt != 0, stream);
  else if (unroll == 8)
    launch_stream_read<8>(p, n, sink, grid, nt != 0, stream);
  else if (unroll == 16)
    launch_stream_read<16>(p, n, sink, grid, nt != 0, stream);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// The decode kernel's loads over a paged F4 cache (one fp16 scale per 32
// values for K and V): k_nib / v_nib [pages][Hkv][8 KB], k_scale / v_scale
// [pages][Hkv][1 KB], page table pt [B][max_pages] whose first n_pages
// entries of every row are valid page ids; `grid` workgroups of 4 waves
// (rounded down to a multiple of B * Hkv); the non-temporal hint when
// nt != 0.  sink: one device word.  0 = launched.
int ceiling_paged_read(const void* k_nib, const void* v_nib, const void* k_scale, const void* v_scale,
                       const int32_t* pt, int B, int max_pages, int n_pages, int Hkv, int grid, int nt,
                       uint32_t* sink, hipStream_t stream) {
  if (!k_nib || !v_nib || !k_scale || !v_scale || !pt || !sink || B <= 0 || Hkv <= 0 || n_pages <= 0 ||
      n_pages > max_pages || grid < B * Hkv)
    return 1;
  const int chunks = grid / (B * Hkv);
  const auto k = static_cast<const u32x4*>(k_nib), v = static_cast<const u32x4*>(v_nib);
  const auto ks = static_cast<const u32x4*>(k_scale), vs = static_cast<const u32x4*>(v_scale);
  if (nt)
    hipLaunchKernelGGL(paged_read_kernel<true>, dim3(chunks * B * Hkv), dim3(256), 0, stream, k, v, ks, vs, pt, B,
                       max_pages, n_pages, Hkv, chunks, sink);
  else
    hipLaunchKernelGGL(paged_read_kernel<false>, dim3(chunks * B * Hkv), dim3(256), 0, stream, k, v, ks, vs, pt, B,
                       max_pages, n_pages, Hkv, chunks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// `grid` workgroups of 4 waves, each wave issuing 4 * iters matrix
// instructions: kind 0 = v_mfma_f32_32x32x16_f16 (32,768 flop each),
// 1 = v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 (131,072), 2 =
// v_mfma_i32_32x32x32_i8 (65,536).  sink: 256 floats of device memory.
// Returns the flops of the launch in *flops; 0 = launched.
int ceiling_mfma(int kind, int iters, int grid, float* sink, double* flops, hipStream_t stream) {
  if (!sink || !flops || iters < 0 || grid <= 0 || kind < 0 || kind > 2) return 1;
  const double per = kind == 0 ? 32768.0 : (kind == 1 ? 131072.0 : 65536.0);
  *flops = per * 4.0 * iters * 4.0 * grid;
  if (kind == 0)
    hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(grid), dim3(256), 0, stream, iters, sink);
  else if (kind == 1)
    hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(grid), dim3(256), 0, stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<2>, dim3(grid), dim3(256), 0, stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
