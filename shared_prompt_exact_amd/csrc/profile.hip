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

// ------------------------------------------------------------ MFMA probe
//
// The matrix-core rate this device sustains: every wave issues back-to-back
// v_mfma_f32_32x32x16_bf16 into four independent accumulators (no memory
// traffic, no dependences between consecutive MFMAs).  Measurement tools
// report it beside the published peak as the achievable ceiling.
namespace {

typedef __bf16 probe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x16 __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(512) mfma_probe_kernel(int iters, float* out) {
  probe_bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)((threadIdx.x & 7) * 0.125f);
    b[i] = (__bf16)(i * 0.0625f);
  }
  probe_f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (out) out[blockIdx.x] = s;   // the launch passes null: nothing is written, the loop stays
}

}  // namespace

extern "C" int64_t dualkv_mfma_probe(int32_t workgroups, int32_t iters, void* stream) {
  if (workgroups < 1 || iters < 1) return -1;
  void* args[] = {&iters, nullptr};
  float* out = nullptr;
  args[1] = &out;
  if (hipLaunchKernel(reinterpret_cast<const void*>(mfma_probe_kernel), dim3(workgroups), dim3(512), args, 0,
                      static_cast<hipStream_t>(stream)) != hipSuccess)
    return -1;
  // 8 waves x iters x 4 MFMAs x 32*32*16*2 flops per workgroup
  return (int64_t)workgroups * 8 * iters * 4 * 32768;
}
