// Opt-in launch profiler.  Between dualkv_profile_start() and
// dualkv_profile_stop() every kernel the library launches is bracketed by
// two HIP events recorded on its own stream; stop() waits for them and
// aggregates the elapsed time per kernel name.  Off (the default), the
// launch path only reads one atomic flag.
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace dualkv {
namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};
struct Stat {
  std::string name;
  int64_t launches;
  double ms;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;
std::vector<Stat> g_stats;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

bool profiling_on() { return g_on.load(std::memory_order_relaxed); }

int profile_begin(const char* name, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_mu);
  Rec r{name, take_event(), take_event()};
  if (r.a == nullptr || r.b == nullptr) return -1;
  if (hipEventRecord(r.a, stream) != hipSuccess) return -1;
  g_recs.push_back(r);
  return (int)g_recs.size() - 1;
}

void profile_end(int slot, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (slot >= 0 && slot < (int)g_recs.size()) (void)hipEventRecord(g_recs[slot].b, stream);
}

}  // namespace dualkv

using namespace dualkv;

extern "C" {

int dualkv_profile_start(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& r : g_recs) {
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  g_stats.clear();
  g_on.store(true);
  return DUALKV_OK;
}

int dualkv_profile_stop(void) {
  g_on.store(false);
  std::lock_guard<std::mutex> lk(g_mu);
  int status = DUALKV_OK;
  for (auto& r : g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      status = DUALKV_ERR_HIP;
    } else {
      bool found = false;
      for (auto& s : g_stats)
        if (s.name == r.name) {
          s.launches += 1;
          s.ms += ms;
          found = true;
        }
      if (!found) g_stats.push_back(Stat{r.name, 1, ms});
    }
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  return status;
}

int dualkv_profile_count(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  return (int)g_stats.size();
}

int dualkv_profile_kernel(int index, const char** name, int64_t* launches, double* total_ms) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (index < 0 || index >= (int)g_stats.size() || !name || !launches || !total_ms)
    return DUALKV_ERR_INVALID_ARGUMENT;
  *name = g_stats[index].name.c_str();
  *launches = g_stats[index].launches;
  *total_ms = g_stats[index].ms;
  return DUALKV_OK;
}

}  // extern "C"
