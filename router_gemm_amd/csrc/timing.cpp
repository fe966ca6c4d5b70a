// timing.cpp -- the optional launch-site timers declared in include/moe_timing.h.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/moe_timing.h"
#include "moe_kernels.h"

namespace {

struct SiteTimer {
  std::atomic<bool> armed{false};
  std::mutex m;
  std::vector<hipEvent_t> start, stop;
  int used = 0;
  bool open = false;  // a "before" was recorded without its "after"
};

SiteTimer g_sites[MOE_SITE_COUNT];

void destroy(SiteTimer &s) {
  for (hipEvent_t e : s.start) (void)hipEventDestroy(e);
  for (hipEvent_t e : s.stop) (void)hipEventDestroy(e);
  s.start.clear();
  s.stop.clear();
  s.used = 0;
  s.open = false;
}

}  // namespace

namespace moe {

void timing_before(int site, hipStream_t st) {
  if (site < 0 || site >= MOE_SITE_COUNT) return;
  SiteTimer &s = g_sites[site];
  if (!s.armed.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> g(s.m);
  if (s.used < (int)s.start.size() && !s.open) {
    (void)hipEventRecord(s.start[s.used], st);
    s.open = true;
  }
}

void timing_after(int site, hipStream_t st) {
  if (site < 0 || site >= MOE_SITE_COUNT) return;
  SiteTimer &s = g_sites[site];
  if (!s.armed.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> g(s.m);
  if (s.open) {
    (void)hipEventRecord(s.stop[s.used], st);
    s.open = false;
    ++s.used;
  }
}

}  // namespace moe

extern "C" {

moe_status moe_timing_arm(int32_t site, int32_t capacity) {
  if (site < 0 || site >= MOE_SITE_COUNT || capacity < 1 || capacity > 100000) return MOE_EINVAL;
  SiteTimer &s = g_sites[site];
  std::lock_guard<std::mutex> g(s.m);
  s.armed.store(false);
  destroy(s);
  s.start.resize(capacity);
  s.stop.resize(capacity);
  for (int i = 0; i < capacity; ++i) {
    if (hipEventCreate(&s.start[i]) != hipSuccess || hipEventCreate(&s.stop[i]) != hipSuccess) {
      s.start.resize(i);
      s.stop.resize(i);
      destroy(s);
      return MOE_EHIP;
    }
  }
  s.armed.store(true);
  return MOE_OK;
}

moe_status moe_timing_read(int32_t site, double *total_ms, int32_t *launches) {
  if (site < 0 || site >= MOE_SITE_COUNT || !total_ms || !launches) return MOE_EINVAL;
  SiteTimer &s = g_sites[site];
  std::lock_guard<std::mutex> g(s.m);
  s.armed.store(false);
  double total = 0.0;
  moe_status st = MOE_OK;
  for (int i = 0; i < s.used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(s.stop[i]) != hipSuccess || hipEventElapsedTime(&ms, s.start[i], s.stop[i]) != hipSuccess) {
      st = MOE_EHIP;
      break;
    }
    total += ms;
  }
  *total_ms = total;
  *launches = s.used;
  destroy(s);
  return st;
}

}  // extern "C"
