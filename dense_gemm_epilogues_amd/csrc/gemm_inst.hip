// One instantiation unit of the fused GEMM kernel: the dtype, B layout and epilog are
// chosen on the compiler command line (-DEP_DT, -DEP_LAY, -DEP_EPI) so that the build can
// compile the instantiations in parallel; every tile configuration is instantiated here.
#include "gemm_kernel.hpp"

#if !defined(EP_DT) || !defined(EP_LAY) || !defined(EP_EPI)
#error "EP_DT, EP_LAY and EP_EPI must be defined"
#endif

#define EP_CAT4(a, b, c, d) a##_##b##_##c##_##d
#define EP_TABLE_NAME(dt, lay, epi) EP_CAT4(kLaunch, dt, lay, epi)

namespace ep {
// Explicit kernel instantiations (emitted in the device pass).
template __global__ void gemm_kernel<EP_DT, EP_LAY, EP_EPI, 0>(GemmArgs);
template __global__ void gemm_kernel<EP_DT, EP_LAY, EP_EPI, 1>(GemmArgs);
template __global__ void gemm_kernel<EP_DT, EP_LAY, EP_EPI, 2>(GemmArgs);
template __global__ void gemm_kernel<EP_DT, EP_LAY, EP_EPI, 3>(GemmArgs);
template __global__ void gemm_kernel<EP_DT, EP_LAY, EP_EPI, 4>(GemmArgs);

#if !defined(__HIP_DEVICE_COMPILE__)
// Host-side launcher table, indexed by tile configuration.
extern const GemmLauncher EP_TABLE_NAME(EP_DT, EP_LAY, EP_EPI)[kNumTileCfgs];
const GemmLauncher EP_TABLE_NAME(EP_DT, EP_LAY, EP_EPI)[kNumTileCfgs] = {
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 0>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 1>,
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 2>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 3>,
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 4>};
#endif
}  // namespace ep
