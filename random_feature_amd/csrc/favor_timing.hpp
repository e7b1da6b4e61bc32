// Kernel launches of the library, with opt-in per-launch timing. When timing is enabled, a launch
// goes through hipExtLaunchKernelGGL with a start and a stop event that the runtime records in the
// kernel's own dispatch, so the interval is the kernel's execution (no separate event packets
// around it); durations are resolved when read. Disabled by default; off, it costs one branch.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace favor {
bool timing_on();
// creates the event pair of one launch and registers it under `name`; false if it could not
bool timing_pair(const char* name, hipEvent_t* start, hipEvent_t* stop);

template <typename... KArgs, typename... Args>
inline void launch(const char* name, void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem,
                   hipStream_t st, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "one argument per kernel parameter");
  hipEvent_t a = nullptr, b = nullptr;
  if (timing_on() && timing_pair(name, &a, &b))
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, a, b, 0u, static_cast<KArgs>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, st, static_cast<KArgs>(args)...);
}
}  // namespace favor
