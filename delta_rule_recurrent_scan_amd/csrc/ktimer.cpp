// Per-kernel timing for measurement harnesses: while enabled, the launchers
// record a HIP event on the launch stream before and after every kernel, and
// osdn_kernel_times() reports the mean duration per kernel name.
//
// This record is the library's one piece of process-global mutable state. It
// is only touched while timing is enabled (a relaxed atomic flag is all a
// launch reads otherwise), and a mutex serialises every access to it.
#include <hip/hip_runtime.h>

#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/osdn.h"
#include "launch.hpp"

namespace osdn {
namespace {

struct Rec {
  const char* name;
  hipEvent_t start, stop;
  bool done;  // the stop event has been recorded
};

struct Timer {
  std::atomic<bool> on{false};
  std::mutex mu;
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  size_t used = 0;

  // (mu held)
  hipEvent_t take() {
    if (used == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};

Timer& timer() {
  static Timer t;
  return t;
}

}  // namespace

int ktimer_before(hipStream_t s, const char* name) {
  Timer& t = timer();
  if (!t.on.load(std::memory_order_relaxed)) return -1;
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on.load(std::memory_order_relaxed)) return -1;
  Rec r{name, t.take(), t.take(), false};
  if (!r.start || !r.stop) return -1;
  if (hipEventRecord(r.start, s) != hipSuccess) return -1;
  t.recs.push_back(r);
  return (int)t.recs.size() - 1;
}

void ktimer_after(hipStream_t s, int handle) {
  if (handle < 0) return;
  Timer& t = timer();
  std::lock_guard<std::mutex> g(t.mu);
  if (handle >= (int)t.recs.size() || t.recs[handle].done) return;
  if (hipEventRecord(t.recs[handle].stop, s) == hipSuccess)
    t.recs[handle].done = true;
}

}  // namespace osdn

extern "C" {

void osdn_kernel_timing(int enable) {
  osdn::Timer& t = osdn::timer();
  std::lock_guard<std::mutex> g(t.mu);
  if (enable) {
    t.recs.clear();
    t.used = 0;
  }
  t.on.store(enable != 0, std::memory_order_relaxed);
}

int osdn_kernel_times(int max, const char** names, int* counts, float* mean_ms) {
  osdn::Timer& t = osdn::timer();
  std::lock_guard<std::mutex> g(t.mu);
  std::vector<const char*> seen;
  std::vector<double> total;
  std::vector<int> n;
  for (const osdn::Rec& r : t.recs) {
    if (!r.done) continue;  // the launch failed after its start event
    if (hipEventSynchronize(r.stop) != hipSuccess) return -1;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return -1;
    size_t i = 0;
    while (i < seen.size() && strcmp(seen[i], r.name) != 0) ++i;
    if (i == seen.size()) {
      seen.push_back(r.name);
      total.push_back(0.0);
      n.push_back(0);
    }
    total[i] += ms;
    n[i] += 1;
  }
  for (size_t i = 0; i < seen.size() && (int)i < max; ++i) {
    if (names) names[i] = seen[i];
    if (counts) counts[i] = n[i];
    if (mean_ms) mean_ms[i] = (float)(total[i] / n[i]);
  }
  return (int)seen.size();
}

}  // extern "C"
