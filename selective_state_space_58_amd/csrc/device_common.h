// Device helpers shared by the library's HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace ssm {

// Workgroup barrier for data exchanged through LDS.  The compiler's barrier
// lowering waits for this wave's outstanding LDS operations only when it
// cannot prove them unnecessary, and it treats LDS traffic of all waves as one
// ordered stream; on gfx950 a value written just before the barrier was
// observed stale by another wave right after it (two workgroups per CU).  So
// wait for this wave's LDS operations (s_waitcnt lgkmcnt(0); vmcnt and expcnt
// left at their maximum) before every barrier that publishes LDS data.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __syncthreads();
}

}  // namespace ssm
