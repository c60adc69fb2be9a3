// Kernel timing: HIP event pairs recorded around the main kernel launch of
// each call while timing is active (host code only).
#include <atomic>
#include <mutex>
#include <vector>

#include "f4kv_internal.h"

namespace f4kv {
namespace {

struct Timer {
  std::mutex mu;
  std::atomic<bool> active{false};
  std::vector<hipEvent_t> start, stop;
  size_t used = 0;
  bool open = false;  // a begin without its end yet
};

Timer g_timers[3];

void destroy_events(Timer& t) {
  for (hipEvent_t e : t.start) (void)hipEventDestroy(e);
  for (hipEvent_t e : t.stop) (void)hipEventDestroy(e);
  t.start.clear();
  t.stop.clear();
  t.used = 0;
  t.open = false;
}

}  // namespace

void timing_begin(int kernel, hipStream_t s) {
  Timer& t = g_timers[kernel];
  if (!t.active.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> g(t.mu);
  if (t.used >= t.start.size()) return;
  if (hipEventRecord(t.start[t.used], s) == hipSuccess) t.open = true;
}

void timing_end(int kernel, hipStream_t s) {
  Timer& t = g_timers[kernel];
  if (!t.active.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.open) return;
  t.open = false;
  if (hipEventRecord(t.stop[t.used], s) == hipSuccess) ++t.used;
}

hipError_t timing_start(int kernel, int max_launches) {
  Timer& t = g_timers[kernel];
  std::lock_guard<std::mutex> g(t.mu);
  t.active.store(false);
  destroy_events(t);
  for (int i = 0; i < max_launches; ++i) {
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t e = hipEventCreate(&a);
    if (e == hipSuccess) {
      e = hipEventCreate(&b);
      if (e != hipSuccess) (void)hipEventDestroy(a);
    }
    if (e != hipSuccess) {
      destroy_events(t);
      return e;
    }
    t.start.push_back(a);
    t.stop.push_back(b);
  }
  t.active.store(true);
  return hipSuccess;
}

hipError_t timing_stop(int kernel, double* total_ms, int64_t* launches) {
  Timer& t = g_timers[kernel];
  std::lock_guard<std::mutex> g(t.mu);
  t.active.store(false);
  double sum = 0.0;
  hipError_t err = hipSuccess;
  for (size_t i = 0; i < t.used; ++i) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(t.stop[i]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start[i], t.stop[i]);
    if (e != hipSuccess) err = e;
    sum += ms;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = static_cast<int64_t>(t.used);
  destroy_events(t);
  return err;
}

}  // namespace f4kv
