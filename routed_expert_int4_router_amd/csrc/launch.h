// Kernel launch with optional in-launch timestamps.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
};

// Per-thread slot. When it holds events, the next launch() on this thread
// records the kernel's own begin and end timestamps into them (taken from the
// dispatch, so the elapsed time is the kernel's execution alone, without the
// gaps that separate event markers would add) and empties the slot.
LaunchEvents& launch_events();

template <class... Params, class... Args>
inline void launch(void (*kernel)(Params...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
  LaunchEvents& ev = launch_events();
  if (ev.start) {
    const LaunchEvents e = ev;
    ev = LaunchEvents{};
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e.start, e.stop, 0u, static_cast<Params>(args)...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, static_cast<Params>(args)...);
  }
}

}  // namespace moe
