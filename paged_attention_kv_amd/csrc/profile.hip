// Opt-in kernel timing for measurement harnesses: while enabled, every kernel
// launch of a class is bracketed by HIP events on its stream, and the elapsed
// times are summed per class when the harness stops recording. Disabled (the
// default), a mark costs one relaxed atomic load.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "kernels.h"
#include "pa.h"

namespace pa {
namespace {

struct Pending {
  int cls;
  hipEvent_t start, stop;
};

std::atomic<bool> g_enabled{false};
std::mutex g_mu;
std::vector<hipEvent_t> g_pool;      // idle events
std::vector<Pending> g_pending;      // recorded launches
hipEvent_t g_open[PA_KERNEL_CLASSES];  // start event of the launch being marked
bool g_has_open[PA_KERNEL_CLASSES];

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

void profile_begin(int cls, hipStream_t stream) {
  if (!g_enabled.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t e = take_event();
  if (!e) return;
  if (hipEventRecord(e, stream) != hipSuccess) {
    g_pool.push_back(e);
    return;
  }
  g_open[cls] = e;
  g_has_open[cls] = true;
}

void profile_end(int cls, hipStream_t stream) {
  if (!g_enabled.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_has_open[cls]) return;
  g_has_open[cls] = false;
  hipEvent_t e = take_event();
  if (!e || hipEventRecord(e, stream) != hipSuccess) {
    g_pool.push_back(g_open[cls]);
    if (e) g_pool.push_back(e);
    return;
  }
  g_pending.push_back({cls, g_open[cls], e});
}

}  // namespace pa

extern "C" {

int pa_profile_begin(void) {
  std::lock_guard<std::mutex> lk(pa::g_mu);
  for (auto& p : pa::g_pending) {
    pa::g_pool.push_back(p.start);
    pa::g_pool.push_back(p.stop);
  }
  pa::g_pending.clear();
  for (int c = 0; c < PA_KERNEL_CLASSES; ++c) pa::g_has_open[c] = false;
  pa::g_enabled.store(true);
  return PA_OK;
}

int pa_profile_end(pa_profile* out) {
  pa::g_enabled.store(false);
  std::lock_guard<std::mutex> lk(pa::g_mu);
  int status = PA_OK;
  if (out) {
    for (int c = 0; c < PA_KERNEL_CLASSES; ++c) {
      out->launches[c] = 0;
      out->total_ms[c] = 0.0;
    }
  }
  for (auto& p : pa::g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
      status = PA_ERR_HIP;
    } else if (out) {
      out->launches[p.cls] += 1;
      out->total_ms[p.cls] += ms;
    }
    pa::g_pool.push_back(p.start);
    pa::g_pool.push_back(p.stop);
  }
  pa::g_pending.clear();
  return status;
}

}  // extern "C"
