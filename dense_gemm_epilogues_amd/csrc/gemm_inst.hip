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
// every tile configuration, in table order
#define EP_FOR_CFGS(X) X(0) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12)
static_assert(kNumTileCfgs == 13, "EP_FOR_CFGS must list every tile configuration");
// Explicit kernel instantiations (emitted in the device pass).
#define EP_INST(c) template __global__ void gemm_kernel<EP_DT, EP_LAY, EP_EPI, c, 0>(GemmArgs);
EP_FOR_CFGS(EP_INST)
// split-K partial kernels depend only on single or dual B: they live in the DEFAULT and the
// SWIGLU unit of each (dtype, layout); the fixup kernels in the K x N unit of each
// (dtype, epilog)
#if EP_EPI == 0 || EP_EPI == 5
#define EP_INST_P(c) template __global__ void gemm_kernel<EP_DT, EP_LAY, EP_EPI, c, 1>(GemmArgs);
EP_FOR_CFGS(EP_INST_P)
#endif
#if EP_LAY == 0
#define EP_INST_F(c) template __global__ void gemm_kernel<EP_DT, 0, EP_EPI, c, 2>(GemmArgs);
EP_FOR_CFGS(EP_INST_F)
#endif

#if !defined(__HIP_DEVICE_COMPILE__)
// Host-side launcher table, indexed by tile configuration.
#define EP_L(c) launch_gemm<EP_DT, EP_LAY, EP_EPI, c>,
extern const GemmLauncher EP_TABLE_NAME(EP_DT, EP_LAY, EP_EPI)[kNumTileCfgs];
const GemmLauncher EP_TABLE_NAME(EP_DT, EP_LAY, EP_EPI)[kNumTileCfgs] = {EP_FOR_CFGS(EP_L)};
#if EP_EPI == 0 || EP_EPI == 5
#define EP_PTABLE_NAME(dt, lay, epi) EP_CAT4(kPartial, dt, lay, epi)
#define EP_LP(c) launch_gemm<EP_DT, EP_LAY, EP_EPI, c, 1>,
extern const GemmLauncher EP_PTABLE_NAME(EP_DT, EP_LAY, EP_EPI)[kNumTileCfgs];
const GemmLauncher EP_PTABLE_NAME(EP_DT, EP_LAY, EP_EPI)[kNumTileCfgs] = {EP_FOR_CFGS(EP_LP)};
#endif
#if EP_LAY == 0
#define EP_FTABLE_NAME(dt, epi) EP_CAT3(kFixup, dt, epi)
#define EP_LF(c) launch_gemm<EP_DT, 0, EP_EPI, c, 2>,
extern const GemmLauncher EP_FTABLE_NAME(EP_DT, EP_EPI)[kNumTileCfgs];
const GemmLauncher EP_FTABLE_NAME(EP_DT, EP_EPI)[kNumTileCfgs] = {EP_FOR_CFGS(EP_LF)};
#endif
#endif
}  // namespace ep
