// lse_merge: fold partial softmax states by log-sum-exp.
//
// FreeToken issue #568 ("Proposed solution" item 2) folds attention over
// device windows by log2-sum-exp.  A partial state of a token range is
// (m, l, o): its max logit, the sum of exp(s - m), and its normalised output.
// Folding C of them:  M = max m_c, w_c = l_c exp(m_c - M), L = sum w_c,
// O = sum w_c o_c / L.  States with l == 0 (empty ranges) carry no weight.
//
// One workgroup per row (D <= 1024): four thread groups each fold a quarter of
// the partial states with 16-byte loads, then fold their results in LDS.
#include "f4kv_internal.h"

namespace f4kv {
namespace {

constexpr int kMergeThreads = 256;
constexpr int kGroups = kMergeThreads / 64;  // partial states are split over 4 thread groups

struct MergeArgs {
  const float* m;
  const float* l;
  const float* o;
  float* out;
  float* out_m;
  float* out_l;
  int32_t C, R, D;
};

// One workgroup per row.  Each of the 4 groups of 64 threads folds a quarter of
// the C partial states (thread = 4 consecutive channels, D <= 256 per pass),
// then the groups fold their results in LDS.
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x, grp = tid >> 6, t = tid & 63;
  __shared__ float s_red[kMergeThreads];
  __shared__ float s_gl[kGroups];
  __shared__ float4_t s_acc[kGroups][64];

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
  const int d4 = a.D / 4;
  const int per = (a.C + kGroups - 1) / kGroups;
  const int c0 = grp * per, c1 = min(a.C, c0 + per);

  for (int j0 = 0; j0 < d4; j0 += 64) {
    const int j = j0 + t;
    float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
    float L = 0.0f;
    if (M != -INFINITY) {
#pragma unroll 4
      for (int c = c0; c < c1; ++c) {
        const int64_t i = static_cast<int64_t>(c) * a.R + r;
        const float lc = a.l[i];
        const float wgt = lc > 0.0f ? lc * __expf(a.m[i] - M) : 0.0f;
        L += wgt;
        if (j < d4 && wgt != 0.0f) acc += wgt * reinterpret_cast<const float4_t*>(a.o + i * a.D)[j];
      }
    }
    s_acc[grp][t] = acc;
    if (t == 0) s_gl[grp] = L;
    __syncthreads();
    if (grp == 0) {
      float Lt = 0.0f;
      float4_t at = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < kGroups; ++q) {
        Lt += s_gl[q];
        at += s_acc[q][t];
      }
      const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
      if (j < d4) reinterpret_cast<float4_t*>(a.out + static_cast<int64_t>(r) * a.D)[j] = at * inv;
      if (t == 0 && j0 == 0) {
        if (a.out_m) a.out_m[r] = Lt > 0.0f ? M : -INFINITY;
        if (a.out_l) a.out_l[r] = Lt;
      }
    }
    __syncthreads();
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
