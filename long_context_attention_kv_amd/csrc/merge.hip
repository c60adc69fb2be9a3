// lse_merge: fold partial softmax states by log-sum-exp.
//
// FreeToken issue #568 ("Proposed solution" item 2) folds attention over
// device windows by log2-sum-exp.  A partial state of a token range is
// (m, l, o): its max logit, the sum of exp(s - m), and its normalised output.
// Folding C of them:  M = max m_c, w_c = l_c exp(m_c - M), L = sum w_c,
// O = sum w_c o_c / L.  States with l == 0 (empty ranges) carry no weight.
//
// One workgroup per row (D <= 1024); each thread owns up to 4 groups of 4
// consecutive channels and streams
// the C partial rows with 16-byte loads.  The C (m, l) pairs are staged in LDS
// in chunks, turned into weights once, and shared by the workgroup.
#include "f4kv_internal.h"

namespace f4kv {
namespace {

constexpr int kMergeThreads = 64;
constexpr int kChunk = 256;

struct MergeArgs {
  const float* m;
  const float* l;
  const float* o;
  float* out;
  float* out_m;
  float* out_l;
  int32_t C, R, D;
};

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ float s_w[kChunk];
  __shared__ float s_red[kMergeThreads];

  // global max over live states
  float mx = -INFINITY;
  for (int c = tid; c < a.C; c += kMergeThreads) {
    const int64_t i = static_cast<int64_t>(c) * a.R + r;
    if (a.l[i] > 0.0f) mx = fmaxf(mx, a.m[i]);
  }
  s_red[tid] = mx;
  __syncthreads();
  for (int w = kMergeThreads / 2; w > 0; w >>= 1) {
    if (tid < w) s_red[tid] = fmaxf(s_red[tid], s_red[tid + w]);
    __syncthreads();
  }
  const float M = s_red[0];
  __syncthreads();

  const int d4 = a.D / 4;
  float4_t acc[4];
  for (int k = 0; k < 4; ++k) acc[k] = float4_t{0.f, 0.f, 0.f, 0.f};
  float L = 0.0f;
  if (M != -INFINITY) {
    for (int c0 = 0; c0 < a.C; c0 += kChunk) {
      const int n = min(kChunk, a.C - c0);
      for (int c = tid; c < n; c += kMergeThreads) {
        const int64_t i = static_cast<int64_t>(c0 + c) * a.R + r;
        const float lc = a.l[i];
        s_w[c] = lc > 0.0f ? lc * __expf(a.m[i] - M) : 0.0f;
      }
      __syncthreads();
      for (int c = 0; c < n; ++c) {
        const float wgt = s_w[c];
        L += wgt;
        if (wgt == 0.0f) continue;
        const float4_t* src = reinterpret_cast<const float4_t*>(
            a.o + (static_cast<int64_t>(c0 + c) * a.R + r) * a.D);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int j = tid + k * kMergeThreads;
          if (j < d4) acc[k] += wgt * src[j];
        }
      }
      __syncthreads();
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  float4_t* dst = reinterpret_cast<float4_t*>(a.out + static_cast<int64_t>(r) * a.D);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j = tid + k * kMergeThreads;
    if (j < d4) dst[j] = acc[k] * inv;
  }
  if (tid == 0) {
    if (a.out_m) a.out_m[r] = L > 0.0f ? M : -INFINITY;
    if (a.out_l) a.out_l[r] = L;
  }
}

}  // namespace

hipError_t launch_merge(const float* m, const float* l, const float* o, int32_t C, int32_t R,
                        int32_t D, float* out, float* out_m, float* out_l, hipStream_t s) {
  if (R == 0) return hipSuccess;
  MergeArgs a{m, l, o, out, out_m, out_l, C, R, D};
  hipLaunchKernelGGL(merge_kernel, dim3(R), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace f4kv
