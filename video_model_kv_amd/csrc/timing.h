// Optional per-launch timing of the library's kernels (for measurement tools):
// while enabled by qkv_timing_enable, every launch made through a TimedLaunch
// scope is bracketed by HIP events recorded on its stream.  Disabled, a scope
// costs one relaxed atomic load.
#pragma once

#include <hip/hip_runtime.h>

namespace qkv {

bool timing_enabled();
// Records the start event on construction and the end event on destruction;
// `name` must be a string literal (it is kept, not copied).
class TimedLaunch {
 public:
  TimedLaunch(const char* name, hipStream_t s);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;

 private:
  int slot_ = -1;
  hipStream_t s_;
};

}  // namespace qkv
