// Internal interface between the C ABI layer (ep_api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

enum Epi : int {
  E_DEFAULT = 0,
  E_BIAS = 1,
  E_RELU_BIAS = 2,
  E_RELU_AUX_BIAS = 3,
  E_DRELU_BGRAD = 4,
  E_SWIGLU = 5,
  E_DSWIGLU = 6,
  E_GELU_BIAS = 7,
  E_GELU_AUX_BIAS = 8,
  E_DGELU_BGRAD = 9,
  E_SWIGLU_AUX = 10,
  E_NUM = 11
};

enum Layout : int { L_KN = 0, L_NK = 1 };
enum DType : int { T_F16 = 0, T_BF16 = 1 };

// Everything a GEMM launch needs; passed by value as the kernel argument.
struct GemmArgs {
  const void* a;
  const void* b;
  const void* b2;       // SWIGLU up weight
  void* d;
  int64_t lda, ldb, ldd;
  int M, N, K;          // N = output columns
  int tiles_m, tiles_n;
  const void* bias;
  uint32_t* aux_out;
  const uint32_t* aux_in;
  int64_t ld_aux;
  float* bgrad_part;    // two-pass: [tiles_m][N] partial column sums; atomic: bgrad itself
  int bgrad_atomic;
  const void* gate;
  const void* up;
  int64_t ld_gu;
  void* d2;
  int64_t ldd2;
  // split-K (see the MODE parameter of gemm_kernel): K-ranges per tile, K-steps per range,
  // the first split tile (tiles before it run whole) and the fp32 partial accumulators
  // [splits][tiles - tail0][BM * BNT]
  int splits, kt_per_split, tail0;
  float* part;
  void* gaux;           // GELU_AUX_BIAS output / DGELU_BGRAD input: pre-activation, element type
  int64_t ld_gaux;
};

// Tile configurations, shared by the kernels (compile-time parameters) and the planner.
//   bm  = workgroup rows; bnt = rows of the B tile held in LDS (output columns per workgroup
//         are bnt, or bnt/2 for the dual-B SwiGLU kernel); bk = k-values per LDS stage;
//   nst = LDS ring stages; occ = workgroups resident per CU (the kernel is compiled so that
//         occ workgroups fit the register file, and its LDS ring fits 160 KiB / occ);
//   vst = 1: tiles go global -> registers -> LDS, one k-step ahead of the LDS ring (2 stages
//         only); 0: global -> LDS directly;
//   mf  = edge of the MFMA output block: 32 (v_mfma_f32_32x32x16, 16 k per instruction) or
//         16 (v_mfma_f32_16x16x32, 32 k per instruction; a quarter of the accumulator
//         traffic per instruction for half the FLOP);
//   cfl = 1 (16x16 only): k-contiguous tiles in the LDS layout that spreads each row's
//         chunks over four slot rows; 0: rows kept whole (16x16: slot rows transposed as
//         4 x 4).  Both keep the 16x16 fragment reads free of bank conflicts; with spread
//         chunks each DMA lane quad fetches 16 bytes of four rows instead of one 64-byte piece.
//   The 64-deep 16x16 configurations keep 128-byte k-contiguous rows, each a whole cache line
//   fetched by 8 consecutive lanes, in a 2-stage ring loaded right after a k-step's barrier;
//   bar2 = 1: two barriers per k-step for every operand layout (0: only where B is N x K;
//   see the POST_BA schedule of gemm_kernel).
struct TileCfg {
  int bm, bnt, bk, nst, occ, vst, mf, cfl, bar2;
  const char* name;
};
constexpr int kNumTileCfgs = 13;
constexpr TileCfg kTileCfgs[kNumTileCfgs] = {
    {256, 256, 32, 4, 1, 0, 32, 0, 0, "256x256x32x4st"},
    {128, 128, 64, 4, 1, 0, 32, 0, 0, "128x128x64x4st"},
    {256, 128, 32, 4, 1, 0, 32, 0, 0, "256x128x32x4st"},
    {128, 256, 32, 4, 1, 0, 32, 0, 0, "128x256x32x4st"},
    {256, 256, 64, 2, 1, 0, 32, 0, 0, "256x256x64x2st"},
    {256, 256, 32, 5, 1, 0, 32, 0, 0, "256x256x32x5st"},
    {256, 128, 32, 3, 2, 0, 32, 0, 0, "256x128x32x3st_2wg"},
    {128, 256, 32, 3, 2, 0, 32, 0, 0, "128x256x32x3st_2wg"},
    {256, 256, 64, 2, 1, 1, 32, 0, 0, "256x256x64x2st_vst"},
    {256, 256, 32, 4, 1, 0, 16, 1, 0, "256x256x32x4st_m16"},
    {256, 256, 32, 4, 1, 0, 16, 0, 0, "256x256x32x4st_m16rows"},
    {256, 256, 64, 2, 1, 0, 16, 0, 0, "256x256x64x2st_m16"},
    {256, 256, 64, 2, 1, 0, 16, 0, 1, "256x256x64x2st_m16_2bar"},
};

typedef void (*GemmLauncher)(const GemmArgs&, hipStream_t);

// [dtype][layout][epi][cfg]; null where not instantiated
GemmLauncher gemm_launcher(int dtype, int layout, int epi, int cfg);
// split-K: the partial kernel depends only on single or dual B, the fixup kernel not on the layout
GemmLauncher gemm_partial_launcher(int dtype, int layout, bool dual, int cfg);
GemmLauncher gemm_fixup_launcher(int dtype, int epi, int cfg);
const char* gemm_kernel_name(int dtype, int layout, int epi, int cfg);

// ---- unfused baseline and reduction kernels (elementwise.hip)
hipError_t launch_bias_add(int dtype, void* z, int64_t ldz, const void* bias, int M, int N, hipStream_t s);
hipError_t launch_relu_pack(int dtype, const void* z, int64_t ldz, void* y, int64_t ldy, uint32_t* aux,
                            int64_t ld_aux, int M, int N, int with_mask, hipStream_t s);
hipError_t launch_mask_apply(int dtype, const void* g, int64_t ldg, const uint32_t* aux, int64_t ld_aux,
                             void* dx, int64_t lddx, int M, int N, hipStream_t s);
hipError_t launch_colsum_partial(int dtype, const void* x, int64_t ldx, float* part, int M, int N,
                                 int rows_per_block, hipStream_t s);
hipError_t launch_bgrad_reduce(const float* part, int nparts, float* bgrad, int N, hipStream_t s);
hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t s);
hipError_t launch_silu_mul(int dtype, const void* g, const void* u, int64_t ldgu, void* h, int64_t ldh,
                           int M, int N, hipStream_t s);
hipError_t launch_gelu_apply(int dtype, void* z, int64_t ldz, void* aux, int64_t ld_aux, int M, int N,
                             hipStream_t s);
hipError_t launch_dgelu_apply(int dtype, void* g, int64_t ldg, const void* aux, int64_t ld_aux, int M, int N,
                              hipStream_t s);
hipError_t launch_dswiglu(int dtype, const void* dh, int64_t lddh, const void* gate, const void* up,
                          int64_t ld_gu, void* dg, int64_t lddg, void* du, int64_t lddu, int M, int N,
                          hipStream_t s);

}  // namespace ep
