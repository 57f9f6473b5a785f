// Optional per-kernel GPU timing with HIP events (benchmark support).
//
// sv_trace_start(capacity) pre-creates 2*capacity events; each later kernel launch made by
// the library (up to `capacity` launches) is given two of them, which the launch stamps with
// the start and end time of that kernel's execution on its stream.  sv_trace_stop() ends
// recording; sv_trace_kernels()/sv_trace_get() wait for the recorded events and report, per
// kernel name, the launch count and total and minimum event-to-event time.  Only host memory
// and HIP event objects are allocated.

#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "sv_internal.h"
#include "sv_launch.h"

#define SV_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

struct Slot {
  const char* name;
  hipEvent_t begin, end;
};

struct Summary {
  std::string name;
  int launches;
  double total_ms, min_ms, max_ms;
};

std::mutex g_mu;
std::atomic<bool> g_on{false};
std::vector<hipEvent_t> g_pool;
std::vector<Slot> g_slots;
size_t g_used = 0;
std::vector<Summary> g_summary;

void destroy_pool() {
  for (hipEvent_t e : g_pool) (void)hipEventDestroy(e);
  g_pool.clear();
  g_slots.clear();
  g_used = 0;
}

}  // namespace

namespace sv {

bool trace_on() { return g_on.load(std::memory_order_relaxed); }

bool trace_slot(const char* name, hipEvent_t* begin, hipEvent_t* end) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || g_used >= g_slots.size()) return false;
  Slot& s = g_slots[g_used++];
  s.name = name;
  *begin = s.begin;
  *end = s.end;
  return true;
}

}  // namespace sv

SV_EXPORT int sv_trace_start(int capacity) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = false;
  destroy_pool();
  g_summary.clear();
  if (capacity <= 0) return 0;
  g_pool.resize(size_t(capacity) * 2);
  for (auto& e : g_pool)
    if (hipEventCreate(&e) != hipSuccess) {
      destroy_pool();
      return -1;
    }
  g_slots.resize(size_t(capacity));
  for (size_t i = 0; i < g_slots.size(); ++i) g_slots[i] = Slot{"", g_pool[2 * i], g_pool[2 * i + 1]};
  g_on = true;
  return 0;
}

SV_EXPORT int sv_trace_stop(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = false;
  return int(g_used);
}

SV_EXPORT int sv_trace_kernels(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = false;
  std::map<std::string, Summary> by;
  for (size_t i = 0; i < g_used; ++i) {
    const Slot& s = g_slots[i];
    if (hipEventSynchronize(s.end) != hipSuccess) return -1;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, s.begin, s.end) != hipSuccess) return -1;
    auto it = by.find(s.name);
    if (it == by.end()) {
      by[s.name] = Summary{s.name, 1, ms, ms, ms};
    } else {
      Summary& m = it->second;
      m.launches += 1;
      m.total_ms += ms;
      if (ms < m.min_ms) m.min_ms = ms;
      if (ms > m.max_ms) m.max_ms = ms;
    }
  }
  g_summary.clear();
  for (auto& kv : by) g_summary.push_back(kv.second);
  return int(g_summary.size());
}

SV_EXPORT int sv_trace_get(int i, char* name, size_t name_len, int* launches, double* total_ms,
                           double* min_ms, double* max_ms) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (i < 0 || size_t(i) >= g_summary.size() || !name || name_len == 0) return -1;
  const Summary& s = g_summary[size_t(i)];
  strncpy(name, s.name.c_str(), name_len - 1);
  name[name_len - 1] = '\0';
  if (launches) *launches = s.launches;
  if (total_ms) *total_ms = s.total_ms;
  if (min_ms) *min_ms = s.min_ms;
  if (max_ms) *max_ms = s.max_ms;
  return 0;
}
