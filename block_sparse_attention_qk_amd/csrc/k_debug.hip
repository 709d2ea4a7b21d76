// Debug builds: the check that fails on purpose, behind sva_debug_selftest,
// so a test can see the plan's debug word reach the host.
#include "kernels.h"

namespace sva {

#ifdef SVA_DEBUG
namespace {

__global__ void debug_selftest_kernel(DevPlan p) {
    SVA_DCHECK(p, threadIdx.x != 0, SVA_DEBUG_SELF);
}

}  // namespace
#endif

hipError_t launch_debug_selftest(const DevPlan& p, hipStream_t s) {
#ifdef SVA_DEBUG
    hipLaunchKernelGGL(debug_selftest_kernel, dim3(1), dim3(64), 0, s, p);
    return hipGetLastError();
#else
    (void)p;
    (void)s;
    return hipErrorNotSupported;
#endif
}

}  // namespace sva
