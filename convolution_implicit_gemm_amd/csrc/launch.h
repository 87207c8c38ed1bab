// Kernel launch for the routes' convolution kernels.
//
// An ordinary launch on the run's stream, except in a timed run
// (fusedconv_run_timed): then the route's first convolution kernel carries
// the caller's start event and its last one the stop event, and
// hipExtLaunchKernelGGL records them from the dispatch itself (the kernel's
// begin and end), so the interval holds the convolution kernels and nothing
// else: no weight preparation, no marker packets.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "internal.h"

namespace fc {

enum LaunchEdge : unsigned { kEdgeNone = 0, kEdgeFirst = 1, kEdgeLast = 2, kEdgeBoth = 3 };

template <typename... KArgs, typename... Args>
inline int launch_conv(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                       const RunArgs& a, unsigned edges, Args... args) {
  hipEvent_t start = (edges & kEdgeFirst) ? (hipEvent_t)a.ev_start : nullptr;
  hipEvent_t stop = (edges & kEdgeLast) ? (hipEvent_t)a.ev_stop : nullptr;
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, (hipStream_t)a.stream, start, stop,
                          0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, (hipStream_t)a.stream, args...);
  return hipPeekAtLastError() == hipSuccess ? FUSEDCONV_OK : FUSEDCONV_ERR_LAUNCH;
}

}  // namespace fc
