// yarn_rope_table / yarn_rope_apply.
//
// Static YaRN (mistral.rs PR #2375, "Changes by area" item 1; ignis
// --model-rope-scaling row): per rotation pair p the frequency blends the
// trained theta^(-2p/n) (below the beta_fast correction dim) with that divided
// by the factor (above the beta_slow dim), linearly in between; the table is
// scaled by the attention factor m, so queries and keys both carry it.  The
// correction dim of a beta is the pair index whose frequency turns beta times
// over the original context.  Positions reach 2^24, so p * theta' and the
// trigonometry are evaluated in fp64 (an fp32 angle is off by ~1e-2 radians at
// a million positions).
#include "f4kv_device.h"

namespace f4kv {
namespace {

struct RopeTableArgs {
  double theta, factor, beta_fast, beta_slow, mscale;
  double lo, hi;  // correction range, already floored / ceiled / clamped
  int32_t rd, n;
  const int32_t* pos;
  float* cos_out;
  float* sin_out;
};

__global__ __launch_bounds__(256) void rope_table_kernel(RopeTableArgs a) {
  const int half = a.rd / 2;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= static_cast<int64_t>(a.n) * half) return;
  const int p = static_cast<int>(gid % half);
  const int64_t i = gid / half;
  const double base = pow(a.theta, -2.0 * p / a.rd);
  double freq = base;
  if (a.factor != 1.0) {
    double ramp = (p - a.lo) / fmax(0.001, a.hi - a.lo);
    ramp = fmin(1.0, fmax(0.0, ramp));
    const double keep = 1.0 - ramp;  // weight of the unscaled frequency
    freq = (base / a.factor) * (1.0 - keep) + base * keep;
  }
  const double ang = static_cast<double>(a.pos[i]) * freq;
  double sn, cs;
  sincos(ang, &sn, &cs);
  a.cos_out[gid] = static_cast<float>(a.mscale * cs);
  a.sin_out[gid] = static_cast<float>(a.mscale * sn);
}

struct RopeApplyArgs {
  const float* c;
  const float* s;
  const void* x;
  void* y;
  int32_t xdt, ydt, T, H, D, rd;
};

__device__ __forceinline__ double load_elem(const void* p, int dt, int64_t i) {
  return dt == F4KV_F32 ? static_cast<double>(static_cast<const float*>(p)[i])
                        : static_cast<double>(bf16_to_f32(static_cast<const uint16_t*>(p)[i]));
}

__device__ __forceinline__ void store_elem(void* p, int dt, int64_t i, double v) {
  if (dt == F4KV_F32)
    static_cast<float*>(p)[i] = static_cast<float>(v);
  else
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(static_cast<float>(v));
}

// One thread per rotation pair, or per pass-through channel, of one (row, head).
__global__ __launch_bounds__(256) void rope_apply_kernel(RopeApplyArgs a) {
  const int half = a.rd / 2;
  const int per_head = half + (a.D - a.rd);
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= static_cast<int64_t>(a.T) * a.H * per_head) return;
  const int e = static_cast<int>(gid % per_head);
  const int64_t th = gid / per_head;
  const int64_t t = th / a.H;
  const int64_t row = th * a.D;
  if (e < half) {
    const double c = a.c[t * half + e];
    const double s = a.s[t * half + e];
    const double x0 = load_elem(a.x, a.xdt, row + e);
    const double x1 = load_elem(a.x, a.xdt, row + e + half);
    double y0, y1;
    rope_rotate_pair(x0, x1, c, s, y0, y1);
    store_elem(a.y, a.ydt, row + e, y0);
    store_elem(a.y, a.ydt, row + e + half, y1);
  } else {
    const int d = a.rd + (e - half);
    store_elem(a.y, a.ydt, row + d, load_elem(a.x, a.xdt, row + d));
  }
}

}  // namespace

hipError_t launch_rope_table(const f4kv_yarn_params& p, double mscale, const int32_t* pos,
                             int32_t n, float* cos_out, float* sin_out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  RopeTableArgs a;
  a.theta = p.theta;
  a.factor = p.factor;
  a.beta_fast = p.beta_fast;
  a.beta_slow = p.beta_slow;
  a.mscale = mscale;
  a.rd = p.rotary_dim;
  a.n = n;
  a.pos = pos;
  a.cos_out = cos_out;
  a.sin_out = sin_out;
  // correction dims: the pair index at which a frequency turns beta times over orig_ctx
  const double two_pi = 6.283185307179586476925286766559;
  auto corr = [&](double beta) {
    return p.rotary_dim * std::log(p.orig_ctx / (two_pi * beta)) / (2.0 * std::log(p.theta));
  };
  a.lo = std::fmax(0.0, std::floor(corr(p.beta_fast)));
  a.hi = std::fmin(static_cast<double>(p.rotary_dim - 1), std::ceil(corr(p.beta_slow)));
  const int64_t total = static_cast<int64_t>(n) * (p.rotary_dim / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_rope_apply(const float* c, const float* sn, const void* x, int32_t xdt,
                             void* y, int32_t ydt, int32_t T, int32_t H, int32_t D, int32_t rd,
                             hipStream_t s) {
  if (T == 0 || H == 0) return hipSuccess;
  RopeApplyArgs a{c, sn, x, y, xdt, ydt, T, H, D, rd};
  const int64_t total = static_cast<int64_t>(T) * H * (rd / 2 + (D - rd));
  hipLaunchKernelGGL(rope_apply_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace f4kv
