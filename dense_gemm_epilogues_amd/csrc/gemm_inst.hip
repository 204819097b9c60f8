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
#define EP_INST(c) template __global__ void gemm_kernel<EP_DT, EP_LAY, EP_EPI, c>(GemmArgs);
EP_INST(0) EP_INST(1) EP_INST(2) EP_INST(3) EP_INST(4) EP_INST(5) EP_INST(6) EP_INST(7)
static_assert(kNumTileCfgs == 8, "instantiate every tile configuration");

#if !defined(__HIP_DEVICE_COMPILE__)
// Host-side launcher table, indexed by tile configuration.
extern const GemmLauncher EP_TABLE_NAME(EP_DT, EP_LAY, EP_EPI)[kNumTileCfgs];
const GemmLauncher EP_TABLE_NAME(EP_DT, EP_LAY, EP_EPI)[kNumTileCfgs] = {
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 0>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 1>,
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 2>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 3>,
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 4>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 5>,
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 6>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 7>};
#endif
}  // namespace ep
