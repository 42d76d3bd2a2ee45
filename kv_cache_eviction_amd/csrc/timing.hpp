// Opt-in per-launch kernel timing (see timing.cpp).
#pragma once

#include <hip/hip_runtime.h>

namespace kvs {

// RAII bracket around one kernel launch: records a start event on construction
// and a stop event on destruction when timing is enabled.
class TimedLaunch {
 public:
  TimedLaunch(const char *name, hipStream_t st);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch &) = delete;
  TimedLaunch &operator=(const TimedLaunch &) = delete;

 private:
  hipStream_t stream_;
  int index_;
};

void timing_enable(int on);
int timing_count();
int timing_read(int i, const char **name, float *ms);
void timing_reset();

}  // namespace kvs
