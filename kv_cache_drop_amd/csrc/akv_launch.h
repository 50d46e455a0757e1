// Kernel launch through the extended launch call, which stamps the timer's
// events from the dispatch itself (no marker packets between kernels).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "akv_internal.h"

namespace akv {

template <typename F, typename... A>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t shared, hipStream_t st, A... args) {
  LaunchEvents& ev = launch_events();
  hipEvent_t start = ev.start;
  ev.start = nullptr;
  hipExtLaunchKernelGGL(kernel, grid, block, shared, st, start, ev.stop, 0u, args...);
}

}  // namespace akv
