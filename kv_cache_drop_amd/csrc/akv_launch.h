// Kernel launches of the library (HIP sources only).  When the pool's timers
// are on, the caller arms a start and a stop event (launch_events()); the
// next launch carries them, so they are stamped by the dispatch itself at the
// kernel's start and end (no marker packets of their own on the stream).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "akv_internal.h"

namespace akv {

template <typename F, typename... Args>
inline void launch_k(F kernel, const dim3& grid, const dim3& block, hipStream_t st, Args... args) {
  LaunchEvents& ev = launch_events();
  hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev.start, ev.stop, 0, args...);
  if (ev.start) ev.used = true;
  ev.start = ev.stop = nullptr;
}

}  // namespace akv
