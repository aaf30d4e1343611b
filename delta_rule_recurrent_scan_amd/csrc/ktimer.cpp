// Per-kernel timing for measurement harnesses: while enabled, the launchers
// record a HIP event on the launch stream before and after every kernel, and
// osdn_kernel_times() reports the mean duration per kernel name.
#include <hip/hip_runtime.h>

#include <string.h>

#include <vector>

#include "../../include/osdn.h"
#include "launch.hpp"

namespace osdn {
namespace {

struct Rec {
  const char* name;
  hipEvent_t start, stop;
};

struct Timer {
  bool on = false;
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  size_t used = 0;

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

void ktimer_before(hipStream_t s, const char* name) {
  Timer& t = timer();
  if (!t.on) return;
  Rec r{name, t.take(), t.take()};
  if (!r.start || !r.stop) return;
  hipEventRecord(r.start, s);
  t.recs.push_back(r);
}

void ktimer_after(hipStream_t s) {
  Timer& t = timer();
  if (!t.on || t.recs.empty()) return;
  hipEventRecord(t.recs.back().stop, s);
}

}  // namespace osdn

extern "C" {

void osdn_kernel_timing(int enable) {
  osdn::Timer& t = osdn::timer();
  t.on = enable != 0;
  if (t.on) {
    t.recs.clear();
    t.used = 0;
  }
}

int osdn_kernel_times(int max, const char** names, int* counts, float* mean_ms) {
  osdn::Timer& t = osdn::timer();
  std::vector<const char*> seen;
  std::vector<double> total;
  std::vector<int> n;
  for (const osdn::Rec& r : t.recs) {
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
