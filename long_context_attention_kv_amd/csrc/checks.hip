// Device-side checks of the values the host cannot validate: context lengths,
// page ids of live pages, slot ids and row offsets live in device memory.  The
// kernels never read or write out of bounds for them (they skip such entries),
// but a caller debugging its own tables wants to know.  When the checks are on
// (f4kv_device_checks), every entry point first launches a small check kernel
// on its own stream that ORs a flag into a per-device word; the word is read
// back and cleared by f4kv_device_check_word.  Off by default: then nothing is
// launched and the entry points cost what they did.
#include <atomic>
#include <mutex>

#include "f4kv_internal.h"

namespace f4kv {
namespace {

// The flag word of each GPU (a device array of the library; host code uses its
// address from hipGetSymbolAddress, never the name).
static __device__ uint32_t check_word;

std::atomic<bool> g_on{false};

hipError_t word_address(uint32_t** ptr) {
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
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_word));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = static_cast<uint32_t*>(addr[dev]);
  return hipSuccess;
}

// One workgroup per sequence: its context length, then the page ids of its
// live pages (tokens [0, ctx), ctx clamped to [0, max_ctx]).
__global__ __launch_bounds__(256) void check_pages_kernel(const int32_t* __restrict__ ctx, int32_t fixed_len,
                                                          const int32_t* __restrict__ pt, int32_t max_pages,
                                                          int32_t max_ctx, int32_t num_pages, uint32_t* word) {
  const int b = blockIdx.x;
  int n = ctx ? ctx[b] : fixed_len;
  if (ctx && (n < 0 || n > max_ctx)) {
    if (threadIdx.x == 0) atomicOr(word, static_cast<uint32_t>(F4KV_CHECK_CONTEXT));
    n = max(0, min(n, max_ctx));
  }
  const int pages = (n + kPage - 1) / kPage;
  const int32_t* row = pt + static_cast<int64_t>(b) * max_pages;
  bool bad = false;
  for (int lp = threadIdx.x; lp < pages; lp += blockDim.x)
    bad |= static_cast<uint32_t>(row[lp]) >= static_cast<uint32_t>(num_pages);
  if (bad) atomicOr(word, static_cast<uint32_t>(F4KV_CHECK_PAGE));
}

__global__ __launch_bounds__(256) void check_slots_kernel(const int32_t* __restrict__ slots, int32_t T,
                                                          int64_t num_slots, uint32_t* word) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int32_t s = slots[t];
  if (s != -1 && (s < 0 || s >= num_slots)) atomicOr(word, static_cast<uint32_t>(F4KV_CHECK_SLOT));
}

// Row offsets of the gather: cu[0] == 0, non-decreasing, each length at most
// max_pages * 64, cu[B] <= total; then the live pages of each sequence.
__global__ __launch_bounds__(256) void check_rows_kernel(const int32_t* __restrict__ cu, int32_t B,
                                                         const int32_t* __restrict__ pt, int32_t max_pages,
                                                         int32_t total, int32_t num_pages, uint32_t* word) {
  const int b = blockIdx.x;
  const int32_t lo = cu[b], hi = cu[b + 1];
  const int64_t len = static_cast<int64_t>(hi) - lo;
  if (threadIdx.x == 0) {
    if ((b == 0 && lo != 0) || len < 0 || len > static_cast<int64_t>(max_pages) * kPage ||
        (b == B - 1 && hi > total))
      atomicOr(word, static_cast<uint32_t>(F4KV_CHECK_ROWS));
  }
  const int pages = len > 0 ? static_cast<int>(min<int64_t>(len, static_cast<int64_t>(max_pages) * kPage) + kPage - 1) / kPage
                            : 0;
  const int32_t* row = pt + static_cast<int64_t>(b) * max_pages;
  bool bad = false;
  for (int lp = threadIdx.x; lp < pages; lp += blockDim.x)
    bad |= static_cast<uint32_t>(row[lp]) >= static_cast<uint32_t>(num_pages);
  if (bad) atomicOr(word, static_cast<uint32_t>(F4KV_CHECK_PAGE));
}

}  // namespace

bool checks_on() { return g_on.load(std::memory_order_relaxed); }

hipError_t check_pages(const int32_t* ctx, int32_t fixed_len, const int32_t* pt, int32_t B, int32_t max_pages,
                       int32_t max_ctx, int32_t num_pages, hipStream_t s) {
  uint32_t* w = nullptr;
  hipError_t e = word_address(&w);
  if (e != hipSuccess || B <= 0) return e;
  hipLaunchKernelGGL(check_pages_kernel, dim3(B), dim3(256), 0, s, ctx, fixed_len, pt, max_pages, max_ctx,
                     num_pages, w);
  return hipGetLastError();
}

hipError_t check_slots(const int32_t* slots, int32_t T, int64_t num_slots, hipStream_t s) {
  uint32_t* w = nullptr;
  hipError_t e = word_address(&w);
  if (e != hipSuccess || T <= 0) return e;
  hipLaunchKernelGGL(check_slots_kernel, dim3((T + 255) / 256), dim3(256), 0, s, slots, T, num_slots, w);
  return hipGetLastError();
}

hipError_t check_rows(const int32_t* cu, int32_t B, const int32_t* pt, int32_t max_pages, int32_t total,
                      int32_t num_pages, hipStream_t s) {
  uint32_t* w = nullptr;
  hipError_t e = word_address(&w);
  if (e != hipSuccess || B <= 0) return e;
  hipLaunchKernelGGL(check_rows_kernel, dim3(B), dim3(256), 0, s, cu, B, pt, max_pages, total, num_pages, w);
  return hipGetLastError();
}

void set_checks(bool on) { g_on.store(on, std::memory_order_relaxed); }

hipError_t read_check_word(uint32_t* out) {
  uint32_t* w = nullptr;
  hipError_t e = word_address(&w);
  if (e != hipSuccess) return e;
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  e = hipMemcpy(out, w, sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  const uint32_t zero = 0;
  return hipMemcpy(w, &zero, sizeof(uint32_t), hipMemcpyHostToDevice);
}

}  // namespace f4kv
