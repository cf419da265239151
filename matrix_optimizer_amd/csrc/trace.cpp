// Launch tracing: when enabled, every kernel launch of muon_step and the stage
// calls carries two HIP events that the runtime records at the kernel's start
// and end (hipExtLaunchKernel), so a caller can read per-kernel durations
// without an external profiler.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/muon.h"
#include "internal.h"

namespace {

struct Rec {
  const char* name;
  hipEvent_t start, stop;
};

std::mutex g_mu;
std::atomic<bool> g_on{false};   // read without the lock on every launch
std::vector<hipEvent_t> g_pool;
std::vector<Rec> g_recs;
size_t g_next = 0;

}  // namespace

namespace muon {

bool trace_take(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  if (!g_on.load(std::memory_order_acquire)) return false;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on.load(std::memory_order_relaxed) || g_next + 2 > g_pool.size()) return false;
  Rec r{name, g_pool[g_next], g_pool[g_next + 1]};
  g_next += 2;
  g_recs.push_back(r);
  *start = r.start;
  *stop = r.stop;
  return true;
}

}  // namespace muon

extern "C" {

muon_status muon_trace_start(int32_t max_launches) {
  if (max_launches < 1) return MUON_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_on) return MUON_ERR_INVALID_ARG;
  for (hipEvent_t e : g_pool) (void)hipEventDestroy(e);
  g_pool.assign(size_t(max_launches) * 2, nullptr);
  for (auto& e : g_pool)
    if (hipEventCreate(&e) != hipSuccess) return MUON_ERR_HIP;
  g_recs.clear();
  g_recs.reserve(max_launches);
  g_next = 0;
  g_on.store(true, std::memory_order_release);
  return MUON_OK;
}

int32_t muon_trace_stop(float* ms, const char** names, int32_t capacity) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on.load(std::memory_order_relaxed)) return -1;
  g_on.store(false, std::memory_order_release);
  int32_t n = 0;
  for (const Rec& r : g_recs) {
    if (n < capacity) {
      float t = -1.f;
      if (hipEventSynchronize(r.stop) == hipSuccess) (void)hipEventElapsedTime(&t, r.start, r.stop);
      if (ms) ms[n] = t;
      if (names) names[n] = r.name;
    }
    ++n;
  }
  for (hipEvent_t e : g_pool) (void)hipEventDestroy(e);
  g_pool.clear();
  g_recs.clear();
  g_next = 0;
  return n;
}

}  // extern "C"
