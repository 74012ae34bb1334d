// One (rows, act dtype, delta dtype, states-per-lane) combination of
// selective-scan kernels.  The build compiles this file once per combination
// with SSM_R, SSM_XB / SSM_DB (1 = bf16, 0 = fp32) and SSM_S set, so the
// instantiations compile in parallel.
#include "scan_impl.h"

#if !defined(SSM_R) || !defined(SSM_XB) || !defined(SSM_DB) || !defined(SSM_S)
#error "SSM_R, SSM_XB, SSM_DB and SSM_S must be defined"
#endif

#define SSM_CAT2(a, b) a##b
#define SSM_CAT(a, b) SSM_CAT2(a, b)
#define SSM_NAME \
  SSM_CAT(SSM_CAT(SSM_CAT(SSM_CAT(launch_scan_r, SSM_R), SSM_CAT(_x, SSM_XB)), SSM_CAT(_d, SSM_DB)), SSM_CAT(_s, SSM_S))

namespace ssm {
hipError_t SSM_NAME(int mode, const ScanArgs& a, dim3 grid, int64_t gpb, hipStream_t st) {
  return scan_dev::launch_scan_variant<SSM_R, SSM_XB != 0, SSM_DB != 0, SSM_S>(mode, a, grid, gpb, st);
}
}  // namespace ssm
