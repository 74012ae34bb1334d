// One (act dtype, delta dtype) pair of selective-scan kernels.  The build
// compiles this file once per pair with SSM_XB / SSM_DB set to 0 or 1
// (bf16 when 1), so the instantiations compile in parallel.
#include "scan_impl.h"

#ifndef SSM_XB
#error "SSM_XB must be defined"
#endif
#ifndef SSM_DB
#error "SSM_DB must be defined"
#endif

#define SSM_CAT2(a, b, c) a##b##c
#define SSM_CAT(a, b, c) SSM_CAT2(a, b, c)

namespace ssm {
hipError_t SSM_CAT(launch_scan_x, SSM_XB, SSM_CAT(_d, SSM_DB, ))(int S, int mode, const ScanArgs& a, dim3 grid,
                                                                 int64_t gpb, hipStream_t st) {
  return scan_dev::launch_scan_variant<SSM_XB != 0, SSM_DB != 0>(S, mode, a, grid, gpb, st);
}
}  // namespace ssm
