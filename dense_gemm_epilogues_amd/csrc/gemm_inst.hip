// One instantiation unit of the fused GEMM kernel: the dtype, B layout and epilog are
// chosen on the compiler command line (-DEP_DT, -DEP_LAY, -DEP_EPI) so that the build can
// compile the instantiations in parallel; every tile configuration is instantiated here.
#include "gemm_kernel.hpp"

#if !defined(EP_DT) || !defined(EP_LAY) || !defined(EP_EPI)
#error "EP_DT, EP_LAY and EP_EPI must be defined"
#endif

#define EP_CAT4(a, b, c, d) a##_##b##_##c##_##d
#define EP_CAT3(a, b, c) EP_CAT3_(a, b, c)
#define EP_CAT3_(a, b, c) a##_##b##_##c
#define EP_TABLE_NAME(dt, lay, epi) EP_CAT4(kLaunch, dt, lay, epi)

namespace ep {
// Explicit kernel instantiations (emitted in the device pass).
#define EP_INST(c) template __global__ void gemm_kernel<EP_DT, EP_LAY, EP_EPI, c, 0>(GemmArgs);
EP_INST(0) EP_INST(1) EP_INST(2) EP_INST(3) EP_INST(4) EP_INST(5) EP_INST(6) EP_INST(7) EP_INST(8)
static_assert(kNumTileCfgs == 9, "instantiate every tile configuration");
// split-K partial kernels depend only on single or dual B: they live in the DEFAULT and the
// SWIGLU unit of each (dtype, layout); the fixup kernels in the K x N unit of each
// (dtype, epilog)
#if EP_EPI == 0 || EP_EPI == 5
#define EP_INST_P(c) template __global__ void gemm_kernel<EP_DT, EP_LAY, EP_EPI, c, 1>(GemmArgs);
EP_INST_P(0) EP_INST_P(1) EP_INST_P(2) EP_INST_P(3) EP_INST_P(4) EP_INST_P(5) EP_INST_P(6) EP_INST_P(7) EP_INST_P(8)
#endif
#if EP_LAY == 0
#define EP_INST_F(c) template __global__ void gemm_kernel<EP_DT, 0, EP_EPI, c, 2>(GemmArgs);
EP_INST_F(0) EP_INST_F(1) EP_INST_F(2) EP_INST_F(3) EP_INST_F(4) EP_INST_F(5) EP_INST_F(6) EP_INST_F(7) EP_INST_F(8)
#endif

#if !defined(__HIP_DEVICE_COMPILE__)
// Host-side launcher table, indexed by tile configuration.
extern const GemmLauncher EP_TABLE_NAME(EP_DT, EP_LAY, EP_EPI)[kNumTileCfgs];
const GemmLauncher EP_TABLE_NAME(EP_DT, EP_LAY, EP_EPI)[kNumTileCfgs] = {
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 0>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 1>,
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 2>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 3>,
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 4>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 5>,
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 6>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 7>,
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 8>};
#if EP_EPI == 0 || EP_EPI == 5
#define EP_PTABLE_NAME(dt, lay, epi) EP_CAT4(kPartial, dt, lay, epi)
extern const GemmLauncher EP_PTABLE_NAME(EP_DT, EP_LAY, EP_EPI)[kNumTileCfgs];
const GemmLauncher EP_PTABLE_NAME(EP_DT, EP_LAY, EP_EPI)[kNumTileCfgs] = {
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 0, 1>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 1, 1>,
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 2, 1>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 3, 1>,
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 4, 1>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 5, 1>,
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 6, 1>, launch_gemm<EP_DT, EP_LAY, EP_EPI, 7, 1>,
    launch_gemm<EP_DT, EP_LAY, EP_EPI, 8, 1>};
#endif
#if EP_LAY == 0
#define EP_FTABLE_NAME(dt, epi) EP_CAT3(kFixup, dt, epi)
extern const GemmLauncher EP_FTABLE_NAME(EP_DT, EP_EPI)[kNumTileCfgs];
const GemmLauncher EP_FTABLE_NAME(EP_DT, EP_EPI)[kNumTileCfgs] = {
    launch_gemm<EP_DT, 0, EP_EPI, 0, 2>, launch_gemm<EP_DT, 0, EP_EPI, 1, 2>,
    launch_gemm<EP_DT, 0, EP_EPI, 2, 2>, launch_gemm<EP_DT, 0, EP_EPI, 3, 2>,
    launch_gemm<EP_DT, 0, EP_EPI, 4, 2>, launch_gemm<EP_DT, 0, EP_EPI, 5, 2>,
    launch_gemm<EP_DT, 0, EP_EPI, 6, 2>, launch_gemm<EP_DT, 0, EP_EPI, 7, 2>,
    launch_gemm<EP_DT, 0, EP_EPI, 8, 2>};
#endif
#endif
}  // namespace ep
