// timing.h -- opt-in HIP-event bracketing of each kernel launch (internal).
#pragma once

#include <hip/hip_runtime.h>

namespace flare {

enum KernelId {
  K_FWD = 0, K_BWD_SCAN, K_BWD_CHUNK, K_BLOCK_STEP, K_SHORTCONV, K_TRI, K_BWD_PRE, K_FWD_PRE, K_FWD_SCAN, K_SHORTCONV_BWD,
  K_SCATTER, K_FWD_PREP,
  K_COUNT
};

// Records a start event on construction and a stop event on destruction, on
// `st`, when timing is enabled; does nothing otherwise.
class TimedLaunch {
 public:
  TimedLaunch(KernelId id, hipStream_t st);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch &) = delete;
  TimedLaunch &operator=(const TimedLaunch &) = delete;

 private:
  KernelId id_;
  hipStream_t st_;
  hipEvent_t start_ = nullptr;
};

}  // namespace flare
