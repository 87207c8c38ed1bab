// Workgroup barrier that orders LDS only.
#pragma once

#include <hip/hip_runtime.h>

namespace fc {

// __syncthreads() is a workgroup-scope release/acquire that also covers
// global memory, so every wave first waits for all of its outstanding global
// loads and stores (vmcnt(0)).  Kernels that keep global loads in flight
// across a barrier (prefetched input, weights one step ahead, stores of the
// previous tile) use this barrier where only LDS data is exchanged.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace fc
