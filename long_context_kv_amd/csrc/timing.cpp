// Per-kernel launch timing with HIP events recorded on the launching stream.
//
// Off by default. When enabled (cart_timing_enable), every kernel launch of
// the library (or, after cart_timing_only, every launch of one kernel name)
// carries a start and a stop event in its dispatch; cart_timing_query
// waits for the recorded events and sums the elapsed times of one kernel
// name. Events are pooled and reused across enable cycles.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "cartattn.h"
#include "timing.hpp"

namespace cartattn {

namespace {

struct Record {
  const char* name;
  hipEvent_t start;
  hipEvent_t stop;
};

std::mutex g_mu;
// Read without the lock on every launch: when timing is off (the normal case)
// a launch costs one relaxed load here and takes no lock.
std::atomic<bool> g_on{false};
std::string g_only;   // when not empty, only launches of this kernel name are timed
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  // Timing-only events: no system-scope fence (cache writeback and
  // invalidation) when they are recorded, which would otherwise stall the
  // stream for several microseconds around every timed launch.
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

void recycle_all() {
  for (auto& r : g_records) {
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_records.clear();
}

}  // namespace

void timing_events(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  *start = nullptr;
  *stop = nullptr;
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on.load(std::memory_order_relaxed)) return;
  if (!g_only.empty() && g_only != name) return;
  Record r{name, take_event(), take_event()};
  if (!r.start || !r.stop) return;
  g_records.push_back(r);
  *start = r.start;
  *stop = r.stop;
}

}  // namespace cartattn

using namespace cartattn;

extern "C" {

int cart_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& r : g_records) hipEventSynchronize(r.stop);
  recycle_all();
  g_on.store(on != 0, std::memory_order_relaxed);
  return CART_OK;
}

int cart_timing_only(const char* kernel) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_only = kernel ? kernel : "";
  return CART_OK;
}

int cart_timing_query(const char* kernel, double* total_ms, int32_t* launches) {
  if (!kernel || !total_ms || !launches) return CART_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_mu);
  double tot = 0.0;
  int n = 0;
  for (auto& r : g_records) {
    if (strcmp(r.name, kernel) != 0) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return CART_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return CART_ERR_HIP;
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return CART_OK;
}

}  // extern "C"
