// Opt-in per-launch timing: when enabled, every kernel launch of the library is
// bracketed by two HIP events recorded on the launch stream. Durations are
// resolved when read. Disabled by default; off, it costs one branch per launch.
#pragma once
#include <hip/hip_runtime_api.h>

namespace favor {
void timing_mark_begin(const char* name, hipStream_t st);
void timing_mark_end(hipStream_t st);

struct TimedLaunch {
  hipStream_t st;
  TimedLaunch(const char* name, hipStream_t s) : st(s) { timing_mark_begin(name, s); }
  ~TimedLaunch() { timing_mark_end(st); }
};
}  // namespace favor

#define FAVOR_TIMED(name, st) ::favor::TimedLaunch favor_timed_launch_guard_(name, st)
