// Optional per-phase kernel timing with HIP events (see zp_profile_enable).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "zp_internal.h"

namespace zp {
namespace {

struct Mark {
  int phase;
  hipEvent_t begin, end;
};

constexpr size_t kPrecreatedEvents = 2048;
std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<hipEvent_t> g_free;  // reusable events
std::vector<Mark> g_marks;       // completed brackets waiting to be read
hipEvent_t g_open[ZP_NUM_PHASES] = {};

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

void prof_begin(int phase, hipStream_t s) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lock(g_mu);
  hipEvent_t e = take_event();
  if (e && hipEventRecord(e, s) == hipSuccess) g_open[phase] = e;
}

void prof_end(int phase, hipStream_t s) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lock(g_mu);
  hipEvent_t b = g_open[phase];
  if (!b) return;
  g_open[phase] = nullptr;
  hipEvent_t e = take_event();
  if (e && hipEventRecord(e, s) == hipSuccess) {
    g_marks.push_back({phase, b, e});
  } else {
    g_free.push_back(b);
    if (e) g_free.push_back(e);
  }
}

}  // namespace zp

extern "C" {

zp_status zp_profile_enable(int32_t on) {
  if (on) {
    // events are created ahead, so that recording them does not create any
    std::lock_guard<std::mutex> lock(zp::g_mu);
    while (zp::g_free.size() + 2 * zp::g_marks.size() < zp::kPrecreatedEvents) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) break;
      zp::g_free.push_back(e);
    }
  }
  zp::g_on.store(on != 0);
  return ZP_OK;
}

zp_status zp_profile_read(double* total_ms, int64_t* launches) {
  zp::clear_error();
  std::lock_guard<std::mutex> lock(zp::g_mu);
  double tot[ZP_NUM_PHASES] = {};
  int64_t cnt[ZP_NUM_PHASES] = {};
  zp_status st = ZP_OK;
  for (auto& m : zp::g_marks) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(m.end);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, m.begin, m.end);
    if (e != hipSuccess) {
      zp::set_error("profile events: %s", hipGetErrorString(e));
      st = ZP_ERR_HIP;
    } else {
      tot[m.phase] += ms;
      cnt[m.phase] += 1;
    }
    zp::g_free.push_back(m.begin);
    zp::g_free.push_back(m.end);
  }
  zp::g_marks.clear();
  for (int i = 0; i < ZP_NUM_PHASES; i++) {
    if (total_ms) total_ms[i] = tot[i];
    if (launches) launches[i] = cnt[i];
  }
  return st;
}

}  // extern "C"
