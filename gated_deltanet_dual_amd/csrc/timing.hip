// timing.hip -- per-launch HIP-event timing behind flare_timing_*().
#include "timing.h"

#include <atomic>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/flare_gdn.h"

namespace flare {

namespace {
const char *const kNames[K_COUNT] = {"gdn_dual_fwd_kernel", "gdn_bwd_scan_kernel",
                                     "gdn_bwd_chunk_kernel", "block_step_kernel",
                                     "shortconv_dual_kernel", "gdn_tri_kernel", "gdn_bwd_pre_kernel",
                                     "gdn_fwd_pre_kernel", "gdn_fwd_scan_kernel", "shortconv_dual_bwd_kernel",
                                     "gdn_scatter_kernel", "gdn_fwd_prep_kernel"};
std::atomic<int> g_on{0};
std::mutex g_mu;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_rec[K_COUNT];
std::vector<hipEvent_t> g_free;  // events of dropped records, reused

hipEvent_t take_event() {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_free.empty()) {
      hipEvent_t e = g_free.back();
      g_free.pop_back();
      return e;
    }
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

TimedLaunch::TimedLaunch(KernelId id, hipStream_t st) : id_(id), st_(st) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  start_ = take_event();
  if (start_ && hipEventRecord(start_, st_) != hipSuccess) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_free.push_back(start_);
    start_ = nullptr;
  }
}

TimedLaunch::~TimedLaunch() {
  if (!start_) return;
  hipEvent_t stop = take_event();
  std::lock_guard<std::mutex> lk(g_mu);
  if (stop && hipEventRecord(stop, st_) == hipSuccess) {
    g_rec[id_].emplace_back(start_, stop);
  } else {
    g_free.push_back(start_);
    if (stop) g_free.push_back(stop);
  }
}

}  // namespace flare

using namespace flare;

extern "C" {

int32_t flare_timing_enable(int32_t on) { return g_on.exchange(on ? 1 : 0); }

double flare_timing_avg_ms(const char *kernel, int64_t *launches) {
  int id = -1;
  for (int i = 0; i < K_COUNT; ++i)
    if (kernel && std::strcmp(kernel, kNames[i]) == 0) id = i;
  if (launches) *launches = 0;
  if (id < 0) return -1.0;
  std::lock_guard<std::mutex> lk(g_mu);
  double sum = 0.0;
  int64_t n = 0;
  for (auto &r : g_rec[id]) {
    float ms = 0.f;
    if (hipEventSynchronize(r.second) != hipSuccess) continue;
    if (hipEventElapsedTime(&ms, r.first, r.second) != hipSuccess) continue;
    sum += ms;
    ++n;
  }
  if (launches) *launches = n;
  return n ? sum / (double)n : -1.0;
}

void flare_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto &v : g_rec) {
    for (auto &r : v) {
      (void)hipEventSynchronize(r.second);
      g_free.push_back(r.first);
      g_free.push_back(r.second);
    }
    v.clear();
  }
}

}  // extern "C"
