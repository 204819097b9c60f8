// C ABI of the fused GEMM + epilogue library: validation, planning, workspace ownership,
// dispatch.  The plan/execute/free split follows the stateful Matmul object described in
// "Fusing Matmul Epilogs with nvmath-python" ("The problem addressed by fused epilogs")
// and the hotdry.top cuBLASLt post (paragraphs 3-6): planning validates, chooses a
// configuration and allocates once; execution only enqueues kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "ep.h"
#include "ep_internal.hpp"
#include "static_scratch.hpp"

namespace ep {

#define EP_DECL_TABLE(dt, lay, epi) extern const GemmLauncher kLaunch_##dt##_##lay##_##epi[kNumTileCfgs];
#define EP_DECL_EPIS(dt, lay)                                                                    \
  EP_DECL_TABLE(dt, lay, 0) EP_DECL_TABLE(dt, lay, 1) EP_DECL_TABLE(dt, lay, 2)                  \
  EP_DECL_TABLE(dt, lay, 3) EP_DECL_TABLE(dt, lay, 4) EP_DECL_TABLE(dt, lay, 5) EP_DECL_TABLE(dt, lay, 6)  \
  EP_DECL_TABLE(dt, lay, 7) EP_DECL_TABLE(dt, lay, 8) EP_DECL_TABLE(dt, lay, 9) EP_DECL_TABLE(dt, lay, 10)
EP_DECL_EPIS(0, 0)
EP_DECL_EPIS(0, 1)
EP_DECL_EPIS(1, 0)
EP_DECL_EPIS(1, 1)
// K x M A (layouts 2 and 3): DEFAULT only
EP_DECL_TABLE(0, 2, 0) EP_DECL_TABLE(0, 3, 0) EP_DECL_TABLE(1, 2, 0) EP_DECL_TABLE(1, 3, 0)
static const GemmLauncher* const kTablesAKM[2][2] = {{kLaunch_0_2_0, kLaunch_0_3_0}, {kLaunch_1_2_0, kLaunch_1_3_0}};

#define EP_ROW(dt, lay)                                                                          \
  {                                                                                              \
    kLaunch_##dt##_##lay##_0, kLaunch_##dt##_##lay##_1, kLaunch_##dt##_##lay##_2,                \
        kLaunch_##dt##_##lay##_3, kLaunch_##dt##_##lay##_4, kLaunch_##dt##_##lay##_5,            \
        kLaunch_##dt##_##lay##_6, kLaunch_##dt##_##lay##_7, kLaunch_##dt##_##lay##_8,            \
        kLaunch_##dt##_##lay##_9, kLaunch_##dt##_##lay##_10                                      \
  }
static const GemmLauncher* const kTables[2][2][E_NUM] = {{EP_ROW(0, 0), EP_ROW(0, 1)},
                                                         {EP_ROW(1, 0), EP_ROW(1, 1)}};

#define EP_DECL_P(dt, lay)                                                  \
  extern const GemmLauncher kPartial_##dt##_##lay##_0[kNumTileCfgs]; \
  extern const GemmLauncher kPartial_##dt##_##lay##_5[kNumTileCfgs];
EP_DECL_P(0, 0) EP_DECL_P(0, 1) EP_DECL_P(1, 0) EP_DECL_P(1, 1)
extern const GemmLauncher kPartial_0_2_0[kNumTileCfgs];
extern const GemmLauncher kPartial_0_3_0[kNumTileCfgs];
extern const GemmLauncher kPartial_1_2_0[kNumTileCfgs];
extern const GemmLauncher kPartial_1_3_0[kNumTileCfgs];
static const GemmLauncher* const kPartialAKM[2][2] = {{kPartial_0_2_0, kPartial_0_3_0},
                                                      {kPartial_1_2_0, kPartial_1_3_0}};
#define EP_DECL_F(dt) EP_DECL_TABLE_F(dt, 0) EP_DECL_TABLE_F(dt, 1) EP_DECL_TABLE_F(dt, 2) \
  EP_DECL_TABLE_F(dt, 3) EP_DECL_TABLE_F(dt, 4) EP_DECL_TABLE_F(dt, 5) EP_DECL_TABLE_F(dt, 6) \
  EP_DECL_TABLE_F(dt, 7) EP_DECL_TABLE_F(dt, 8) EP_DECL_TABLE_F(dt, 9) EP_DECL_TABLE_F(dt, 10)
#define EP_DECL_TABLE_F(dt, epi) extern const GemmLauncher kFixup_##dt##_##epi[kNumTileCfgs];
EP_DECL_F(0) EP_DECL_F(1)
// [dtype][layout][single B, dual B]
static const GemmLauncher* const kPartialTables[2][2][2] = {
    {{kPartial_0_0_0, kPartial_0_0_5}, {kPartial_0_1_0, kPartial_0_1_5}},
    {{kPartial_1_0_0, kPartial_1_0_5}, {kPartial_1_1_0, kPartial_1_1_5}}};
static const GemmLauncher* const kFixupTables[2][E_NUM] = {
    {kFixup_0_0, kFixup_0_1, kFixup_0_2, kFixup_0_3, kFixup_0_4, kFixup_0_5, kFixup_0_6, kFixup_0_7, kFixup_0_8,
     kFixup_0_9, kFixup_0_10},
    {kFixup_1_0, kFixup_1_1, kFixup_1_2, kFixup_1_3, kFixup_1_4, kFixup_1_5, kFixup_1_6, kFixup_1_7, kFixup_1_8,
     kFixup_1_9, kFixup_1_10}};

GemmLauncher gemm_partial_launcher(int dtype, int layout, bool dual, int cfg) {
  if (dtype < 0 || dtype > 1 || layout < 0 || layout > 3 || cfg < 0 || cfg >= kNumTileCfgs) return nullptr;
  if (layout >= 2) return dual ? nullptr : kPartialAKM[dtype][layout - 2][cfg];
  return kPartialTables[dtype][layout][dual ? 1 : 0][cfg];
}

GemmLauncher gemm_fixup_launcher(int dtype, int epi, int cfg) {
  if (dtype < 0 || dtype > 1 || epi < 0 || epi >= E_NUM || cfg < 0 || cfg >= kNumTileCfgs) return nullptr;
  return kFixupTables[dtype][epi][cfg];
}

GemmLauncher gemm_launcher(int dtype, int layout, int epi, int cfg) {
  if (dtype < 0 || dtype > 1 || layout < 0 || layout > 3 || epi < 0 || epi >= E_NUM || cfg < 0 ||
      cfg >= kNumTileCfgs)
    return nullptr;
  if (layout >= 2) return epi == E_DEFAULT ? kTablesAKM[dtype][layout - 2][cfg] : nullptr;
  return kTables[dtype][layout][epi][cfg];
}

static const char* kEpiNames[E_NUM] = {"DEFAULT", "BIAS",     "RELU_BIAS",     "RELU_AUX_BIAS", "DRELU_BGRAD",
                                       "SWIGLU",  "DSWIGLU", "GELU_BIAS",     "GELU_AUX_BIAS", "DGELU_BGRAD",
                                       "SWIGLU_AUX"};

}  // namespace ep

using namespace ep;

static_assert(EP_NOALLOC_SCRATCH_BYTES == kStaticScratchBytes, "the header states the scratch size");

namespace {

constexpr uint64_t kMagic = 0x6570706c616e3031ULL;  // "epplan01"
constexpr uint64_t kDead = 0xdeadbeefdeadbeefULL;
constexpr int64_t kMaxDim = (int64_t)1 << 31;
// threads per workgroup of the GEMM kernels (kThreads of gemm_kernel.hpp)
constexpr int64_t kGemmWgThreads = 256;
constexpr int64_t kMaxLd = (int64_t)1 << 22;

thread_local std::string t_last_error;

ep_status fail(ep_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  t_last_error = buf;
  return s;
}

struct UnfusedBufs {
  void* z = nullptr;   // GEMM result (DEFAULT epilog) in the element type
  void* z2 = nullptr;  // second GEMM result (SwiGLU up branch)
  int64_t ldz = 0;
};

}  // namespace

struct ep_plan_s {
  uint64_t magic;
  ep_shape shape;
  ep_dtype dtype;
  ep_epilog epilog;
  ep_epilog_io io;
  ep_options opt;
  int device;
  int cfg;
  GemmArgs args;       // fused launch (or the DEFAULT GEMM of the unfused path)
  GemmArgs args2;      // unfused SwiGLU: the up-branch GEMM
  GemmLauncher launch;
  GemmLauncher launch_partial, launch_fixup;  // split-K (splits > 1)
  int splits;
  void* workspace;     // single allocation owned by the plan (NULL for a plan on the stack)
  size_t workspace_bytes;
  size_t part_bytes, z_bytes, kpart_bytes;  // its pieces: bgrad partials, unfused intermediates
                                            // (two of z_bytes), split-K partials
  float* part;         // bgrad partials (two-pass)
  int nparts;
  UnfusedBufs uf;
  int colsum_rows;     // unfused colsum rows per partial block
};

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The dual-B kernel with a K x N B operand keeps the gate and up columns in separate
// 128-column LDS sub-tiles, which needs a 256-row B tile.
bool cfg_allowed(int cfg, bool dual, ep_b_layout lay) {
  return !(dual && lay == EP_B_KN && kTileCfgs[cfg].bnt < 256);
}
// The 64-deep 16x16 configuration loads whole k-steps with no per-lane bounds on k, so it runs
// only where K is a multiple of 64.
bool cfg_fits_k(int cfg, int64_t k) {
  return !(kTileCfgs[cfg].mf == 16 && kTileCfgs[cfg].bk == 64 && k % 64 != 0);
}

int choose_cfg(int64_t m, int64_t n, bool dual, ep_b_layout lay, int cus) {
  // Estimated time ~ rounds of resident tiles x work per tile / relative efficiency.
  // Relative main-loop efficiency of each configuration, measured on MI355X at full-chip
  // shapes (fp16/bf16, both B layouts, every epilog): 256x256x32 with 4 stages is the
  // fastest wherever it fills the chip.
  // (the configuration run for a 256x256 tile, 16x16x32 or register-staged, is chosen by
  // pick_cfg's rule, not by this model)
  static const double kEff[kNumTileCfgs] = {1.0, 0.70, 0.80, 0.80, 0.85, 0.97, 0.80, 0.82, 0.0, 0.0, 0.0, 0.0, 0.0};
  int best = 0;
  double best_t = 1e300;
  for (int c = 0; c < kNumTileCfgs; ++c) {
    if (!cfg_allowed(c, dual, lay) || kEff[c] <= 0.0) continue;
    const int64_t bn = dual ? kTileCfgs[c].bnt / 2 : kTileCfgs[c].bnt;
    const int64_t tiles = ((m + kTileCfgs[c].bm - 1) / kTileCfgs[c].bm) * ((n + bn - 1) / bn);
    const int64_t slots = (int64_t)cus * kTileCfgs[c].occ;
    const int64_t rounds = (tiles + slots - 1) / slots;
    const double t = (double)rounds * (double)(kTileCfgs[c].bm * bn) * kTileCfgs[c].occ / kEff[c];
    if (t < best_t * 0.999) {
      best_t = t;
      best = c;
    }
  }
  return best;
}

// The 256x256 tile is run with 16x16x32 MFMAs: on MI355X the card runs these at a higher
// clock for the same power, and the kernel measured 2-7 % faster than the 32x32x16 form for
// both B layouts, every workload shape from one round of tiles (4096^3) to 64 (65536 x 8192
// x 16384), N x K operands whose 32 KiB row stride makes L2 sets conflict, the split-K down
// GEMM and the dSwiGLU GEMM.  Of its two LDS layouts for k-contiguous tiles (both free of
// bank conflicts), whole rows (configuration 10) measured faster wherever B is given N x K
// (65536 x 16384 x 8192 backward 1173 -> 1213 TFLOP/s sustained, 16384 x 32768 x 4096
// 1235 -> 1272, the 2048 x 5120 x 17408 down GEMM 0.396 -> 0.353 ms; 4096^3 on par), and
// spread chunks (configuration 9) where only A is k-contiguous (4096^3 forward 1174 -> 1190,
// 65536 x 8192 x 16384 forward 1205 -> 1231).  The dual-B SwiGLU GEMM with N x K weights
// at few rounds had been faster on the 64-deep register-staged 32x32 configuration, whose
// loads arrive as whole 128-byte lines; since the 16x16 kernels load k-steps in line-sharing
// pairs, configuration 10 is ahead there too (M 2048 / 4096, H 5120, I 17408: 0.730 ->
// 0.706 ms, 1.209 -> 1.161 ms).  The exception is a single-B GEMM with N x K weights that
// fills less than one round of CUs (long-K GEMMs such as the SwiGLU down and dx GEMMs, 160
// tiles): there the 64-deep register-staged 32x32 configuration measured 7-10% faster with
// cold operands (2048 x 5120 x 17408: 0.386 -> 0.351 ms unsplit; 2048 x 5120 x 34816: 0.746
// -> 0.676 ms with 3 splits).  The unfused path's GEMM takes the tile the fused epilog would.
//
// 64-deep k-steps with 128-byte row pieces (configuration 11) replace both 32-deep 16x16
// configurations wherever K is a multiple of 64: each row piece is then a whole cache line
// fetched by 8 consecutive lanes (the 32-deep ones fetch half lines, which stalled the texture
// addresser on the L1 4-12 times as often as a library GEMM of the same shape), the loop needs
// 5 VALU instructions per 64 k instead of 38-51 and one or two barriers per 64 k instead of two
// (B K x N / N x K; see configuration 12 below).  Measured at
// 65536 x 8192 x 16384 (B K x N) 14.50 -> 13.85 ms, 65536 x 16384 x 8192 (B N x K)
// 14.54 -> 13.72 ms, 4096^3 120.9 -> 116.1 us (K x N) and 114.6 -> 108.3 us (N x K).  It
// also takes over the single-B N x K GEMMs under one round once they are split: with the
// split-K fixup reading its partials in batches, the 2048 x 5120 x 17408 down GEMM runs in
// 0.316 ms on it with 3 splits against 0.339 ms for the register-staged configuration's best
// (3 splits) and 0.357 ms unsplit; the register-staged one remains the choice there when K is
// not a multiple of 64.
//
// Where B is given K x N, the 64-deep form with two barriers per k-step (configuration 12)
// is taken except for long K loops over many rounds: 2-7 % faster on the SwiGLU-MLP GEMMs (K
// 5120 at M 2048 and 16384, the split dx GEMM at K 34816) and the square layer, 0.5-1 %
// slower on the 65536 x 8192 x 16384 forward (K 16384, 32 rounds).  With A given K x M as
// well (the weight gradients, K 2048) it measured 2-2.5 % faster at 5120 x 17408 and
// 34816 x 5120 and on par at 17408 x 5120; with A K x M and B N x K, 0.2-0.6 % slower.  With
// B given N x K (A M x K) the two measured equal within 0.1 % at 65536 x 16384 x 8192, 4096^3
// and 16384^2 x 4096 (A/B runs alternating their order), so those keep configuration 11.
constexpr int kVstCfg = 8;
constexpr int kM16SpreadCfg = 9;
constexpr int kM16RowsCfg = 10;
constexpr int kM16DeepCfg = 11;
constexpr int kM16Deep2BarCfg = 12;
int pick_cfg(const ep_shape* s, int model_cfg, int cus, bool dual) {
  if (model_cfg != 0) return model_cfg;
  const int64_t tiles = ((s->m + 255) / 256) * ((s->n + 255) / 256);
  if (cfg_fits_k(kM16DeepCfg, s->k) && s->b_layout == EP_B_KN && !(s->k >= 8192 && tiles >= 8 * (int64_t)cus))
    return kM16Deep2BarCfg;
  if (cfg_fits_k(kM16DeepCfg, s->k)) return kM16DeepCfg;
  if (!dual && s->a_layout == EP_A_MK && s->b_layout == EP_B_NK && tiles < cus) return kVstCfg;
  return s->b_layout == EP_B_NK ? kM16RowsCfg : kM16SpreadCfg;
}

// Split-K: how many K ranges per tile, and over which tiles.  Times are modelled in
// microseconds: a tile's K loop takes about 0.8 us per 32 k-values with every CU busy (the
// 64-deep 16x16 kernels at MI355X's clock under load: 65536 x 8192 x 16384 and the SwiGLU-MLP
// GEMMs), a round of resident tiles takes one tile time, and each split tile adds the write
// and the read of its fp32 partial (BM * BNT * 4 bytes each way) at about 3.6 TB/s, plus the
// fixup launch.  Two forms:
//   * grids under one round: every tile is split (2048 x 5120 at K 17408 / 34816, 160 tiles:
//     3 splits measured 0.364 -> 0.316 ms and 0.857 -> 0.639 ms; each further split costs
//     about 23 us there, as the model says);
//   * grids with a partly filled last round: the tiles of the whole rounds run unsplit and
//     only the last round's tiles are split, which costs a fixed ~35 us more (two more
//     launches and the fixup's epilog): 2048 x 17408 x 5120 dSwiGLU (2 rounds + 32 tiles)
//     0.428 -> 0.409 ms with 4 splits, the dual-B SwiGLU forward at M 2048 (4 rounds + 64)
//     0.601 -> 0.583 ms with 3; the short-K (2048) weight-gradient GEMMs lose with any split.
// A split is taken when the model expects it at least 3 % faster (one more range than the
// best so far only when 1 % faster still), and only with at least 16 k-steps per range.
struct SplitChoice {
  int splits, tail0;  // K ranges per split tile; tiles [0, tail0) run unsplit
};
SplitChoice choose_splits(int64_t tiles, int slots, int kt, int cfg) {
  const double tile_us = kt * (kTileCfgs[cfg].bk / 32.0) * 0.8;
  const double part_us = 2.0 * kTileCfgs[cfg].bm * kTileCfgs[cfg].bnt * 4.0 / 3.6e6;  // per split tile
  auto rounds = [&](int64_t n) { return (double)((n + slots - 1) / slots); };
  const int64_t whole = tiles / slots * slots, rem = tiles - whole;
  SplitChoice best{1, 0};
  double best_t = rounds(tiles) * tile_us * 0.97;
  for (int sp = 2; sp <= EP_MAX_SPLIT_K; ++sp) {
    if (kt / sp < 16) break;
    double t;
    SplitChoice c;
    if (whole == 0) {
      t = rounds(tiles * sp) / sp * tile_us + sp * tiles * part_us + 10.0;
      c = {sp, 0};
    } else if (rem > 0) {
      t = (whole / slots) * tile_us + rounds(rem * sp) / sp * tile_us + sp * rem * part_us + 35.0;
      c = {sp, (int)whole};
    } else {
      break;  // whole rounds: nothing to gain
    }
    if (t < (best.splits > 1 ? best_t * 0.99 : best_t)) {  // more ranges only for a clear gain
      best_t = t;
      best = c;
    }
  }
  return best;
}

// The integer a caller stored in an enum-typed field.  A C caller may store any int there;
// loading a value outside the enumerators as the enum type is undefined in C++, so the
// checks read the raw int.
template <class E>
int raw_enum(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "ABI enums are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

ep_status validate(const ep_shape* s, ep_dtype dtype, ep_epilog epi, const ep_epilog_io* io,
                   const ep_options* opt) {
  if (!s) return fail(EP_ERR_INVALID_ARG, "shape is NULL");
  if (!io) return fail(EP_ERR_INVALID_ARG, "epilog_io is NULL");
  if (dtype != EP_F16 && dtype != EP_BF16) return fail(EP_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if ((int)epi < 0 || (int)epi >= E_NUM) return fail(EP_ERR_UNSUPPORTED, "unknown epilog %d", (int)epi);
  if (raw_enum(s->b_layout) != EP_B_KN && raw_enum(s->b_layout) != EP_B_NK)
    return fail(EP_ERR_UNSUPPORTED, "unknown B layout %d", raw_enum(s->b_layout));
  if (raw_enum(s->a_layout) != EP_A_MK && raw_enum(s->a_layout) != EP_A_KM)
    return fail(EP_ERR_UNSUPPORTED, "unknown A layout %d", raw_enum(s->a_layout));
  if (s->a_layout == EP_A_KM && epi != EP_EPILOG_DEFAULT)
    return fail(EP_ERR_UNSUPPORTED, "a K x M A operand is supported with the DEFAULT epilog only");
  if (s->m < 1 || s->n < 1 || s->k < 1) return fail(EP_ERR_INVALID_ARG, "m, n, k must be >= 1");
  if (s->m >= kMaxDim || s->n >= kMaxDim) return fail(EP_ERR_UNSUPPORTED, "m and n must be < 2^31");
  // the kernels form k-offsets as (k-step index) x (k-step depth <= 64) in 32 bits, including
  // the index one past the last k-step
  if (s->k > kMaxDim - 64) return fail(EP_ERR_UNSUPPORTED, "k must be <= 2^31 - 64");
  if (s->n % 8 || s->k % 8) return fail(EP_ERR_UNSUPPORTED, "n and k must be multiples of 8");
  if (s->a_layout == EP_A_KM && s->m % 8) return fail(EP_ERR_UNSUPPORTED, "a K x M A needs m % 8 == 0");
  if (opt) {
    if (raw_enum(opt->path) != EP_PATH_FUSED && raw_enum(opt->path) != EP_PATH_UNFUSED)
      return fail(EP_ERR_INVALID_ARG, "unknown path %d", raw_enum(opt->path));
    if (raw_enum(opt->bgrad_mode) != EP_BGRAD_TWO_PASS && raw_enum(opt->bgrad_mode) != EP_BGRAD_ATOMIC)
      return fail(EP_ERR_INVALID_ARG, "unknown bgrad mode %d", raw_enum(opt->bgrad_mode));
    if (opt->tile_cfg < -1 || opt->tile_cfg >= kNumTileCfgs)
      return fail(EP_ERR_INVALID_ARG, "tile_cfg %d out of range", opt->tile_cfg);
    if (opt->split_k < 0 || opt->split_k > EP_MAX_SPLIT_K)
      return fail(EP_ERR_INVALID_ARG, "split_k %d out of range [0, %d]", opt->split_k, EP_MAX_SPLIT_K);
    if (opt->path == EP_PATH_UNFUSED && opt->split_k > 1)
      return fail(EP_ERR_UNSUPPORTED, "split_k applies to the fused path only");
    if (opt->split_tail != 0 && opt->split_tail != 1)
      return fail(EP_ERR_INVALID_ARG, "split_tail must be 0 or 1");
    if (opt->autotune != 0 && opt->autotune != 1)
      return fail(EP_ERR_INVALID_ARG, "autotune must be 0 or 1");
    if (opt->autotune && (opt->path != EP_PATH_FUSED || opt->tile_cfg >= 0 || opt->split_k != 0))
      return fail(EP_ERR_INVALID_ARG, "autotune needs the fused path, tile_cfg -1 and split_k 0");
  }
  // operand pointers
  if (!s->a || !s->b || !s->d) return fail(EP_ERR_INVALID_ARG, "a, b and d must be non-NULL");
  if (!aligned(s->a, 16) || !aligned(s->b, 16) || !aligned(s->d, 16))
    return fail(EP_ERR_INVALID_ARG, "a, b and d must be 16-byte aligned");
  const int64_t brow = s->b_layout == EP_B_KN ? s->n : s->k;
  const int64_t arow = s->a_layout == EP_A_KM ? s->m : s->k;
  if (s->lda < arow || s->lda % 8 || s->lda >= kMaxLd)
    return fail(EP_ERR_INVALID_ARG, "lda must be a multiple of 8 in [row length, 2^22)");
  if (s->ldb < brow || s->ldb % 8 || s->ldb >= kMaxLd)
    return fail(EP_ERR_INVALID_ARG, "ldb must be a multiple of 8 in [row length, 2^22)");
  if (s->ldd < s->n || s->ldd % 8 || s->ldd >= kMaxLd)
    return fail(EP_ERR_INVALID_ARG, "ldd must be a multiple of 8 in [n, 2^22)");

  const bool wants_bias = epi == EP_EPILOG_BIAS || epi == EP_EPILOG_RELU_BIAS || epi == EP_EPILOG_RELU_AUX_BIAS ||
                          epi == EP_EPILOG_GELU_BIAS || epi == EP_EPILOG_GELU_AUX_BIAS;
  const bool wants_aux_out = epi == EP_EPILOG_RELU_AUX_BIAS;
  const bool wants_aux_in = epi == EP_EPILOG_DRELU_BGRAD;
  const bool wants_bgrad = epi == EP_EPILOG_DRELU_BGRAD || epi == EP_EPILOG_DGELU_BGRAD;
  const bool wants_gaux = epi == EP_EPILOG_GELU_AUX_BIAS || epi == EP_EPILOG_DGELU_BGRAD;
  const bool wants_b2 = epi == EP_EPILOG_SWIGLU || epi == EP_EPILOG_SWIGLU_AUX;
  const bool wants_gu = epi == EP_EPILOG_DSWIGLU;
  const bool wants_d2 = wants_gu || epi == EP_EPILOG_SWIGLU_AUX;
  if (wants_bias != (io->bias != nullptr))
    return fail(EP_ERR_INVALID_ARG, wants_bias ? "bias is required" : "bias must be NULL for this epilog");
  if (wants_aux_out != (io->relu_aux != nullptr))
    return fail(EP_ERR_INVALID_ARG, wants_aux_out ? "relu_aux output is required" : "relu_aux must be NULL");
  if (wants_aux_in != (io->relu_aux_in != nullptr))
    return fail(EP_ERR_INVALID_ARG, wants_aux_in ? "relu_aux_in is required" : "relu_aux_in must be NULL");
  if (wants_bgrad != (io->bgrad != nullptr))
    return fail(EP_ERR_INVALID_ARG, wants_bgrad ? "bgrad output is required" : "bgrad must be NULL");
  if (wants_gaux != (io->gelu_aux != nullptr))
    return fail(EP_ERR_INVALID_ARG, wants_gaux ? "gelu_aux is required" : "gelu_aux must be NULL for this epilog");
  if (wants_gaux && !aligned(io->gelu_aux, 16)) return fail(EP_ERR_INVALID_ARG, "gelu_aux must be 16-byte aligned");
  if (wants_bgrad && !aligned(io->bgrad, 16)) return fail(EP_ERR_INVALID_ARG, "bgrad must be 16-byte aligned");
  if (wants_gaux) {
    const int64_t ld = io->ld_gelu_aux == 0 ? s->n : io->ld_gelu_aux;
    if (ld < s->n || ld % 8 || ld >= kMaxLd)
      return fail(EP_ERR_INVALID_ARG, "ld_gelu_aux must be a multiple of 8 in [n, 2^22)");
  } else if (io->ld_gelu_aux != 0) {
    return fail(EP_ERR_INVALID_ARG, "ld_gelu_aux must be 0 for this epilog");
  }
  if (wants_b2 != (io->b2 != nullptr))
    return fail(EP_ERR_INVALID_ARG, wants_b2 ? "b2 (up weight) is required" : "b2 must be NULL");
  if (wants_gu != (io->gate != nullptr) || wants_gu != (io->up != nullptr))
    return fail(EP_ERR_INVALID_ARG, wants_gu ? "gate and up are required" : "gate and up must be NULL");
  if (wants_d2 != (io->d2 != nullptr))
    return fail(EP_ERR_INVALID_ARG, wants_d2 ? "d2 is required" : "d2 must be NULL for this epilog");
  if (wants_d2 && !aligned(io->d2, 16)) return fail(EP_ERR_INVALID_ARG, "d2 must be 16-byte aligned");
  if (wants_bias && !aligned(io->bias, 16)) return fail(EP_ERR_INVALID_ARG, "bias must be 16-byte aligned");
  if (wants_b2 && !aligned(io->b2, 16)) return fail(EP_ERR_INVALID_ARG, "b2 must be 16-byte aligned");
  if (wants_gu && (!aligned(io->gate, 16) || !aligned(io->up, 16) || !aligned(io->d2, 16)))
    return fail(EP_ERR_INVALID_ARG, "gate, up and d2 must be 16-byte aligned");
  if ((wants_aux_out && !aligned(io->relu_aux, 4)) || (wants_aux_in && !aligned(io->relu_aux_in, 4)) ||
      (wants_aux_in && !aligned(io->bgrad, 16)))
    return fail(EP_ERR_INVALID_ARG, "relu_aux must be 4-byte and bgrad 16-byte aligned");
  if (wants_aux_out || wants_aux_in) {
    const int64_t nw = (s->n + 31) / 32;
    const int64_t ld = io->ld_aux == 0 ? nw : io->ld_aux;
    if (ld < nw || ld >= kMaxLd) return fail(EP_ERR_INVALID_ARG, "ld_aux must be >= ceil(n/32)");
  } else if (io->ld_aux != 0) {
    return fail(EP_ERR_INVALID_ARG, "ld_aux must be 0 for this epilog");
  }
  if (wants_gu) {
    const int64_t ldgu = io->ld_gu == 0 ? s->n : io->ld_gu;
    if (ldgu < s->n || ldgu % 8 || ldgu >= kMaxLd) return fail(EP_ERR_INVALID_ARG, "ld_gu must be a multiple of 8 in [n, 2^22)");
  } else if (io->ld_gu != 0) {
    return fail(EP_ERR_INVALID_ARG, "ld_gu must be 0 for this epilog");
  }
  if (wants_d2) {
    const int64_t d2w = wants_gu ? s->n : 2 * s->n;  // DSWIGLU: d_up; SWIGLU_AUX: [gate | up]
    const int64_t ldd2 = io->ldd2 == 0 ? (wants_gu ? s->ldd : d2w) : io->ldd2;
    if (ldd2 < d2w || ldd2 % 8 || ldd2 >= kMaxLd)
      return fail(EP_ERR_INVALID_ARG, "ldd2 must be a multiple of 8 in [d2 row length, 2^22)");
  } else if (io->ldd2 != 0) {
    return fail(EP_ERR_INVALID_ARG, "ldd2 must be 0 for this epilog");
  }
  if (opt && opt->bgrad_mode == EP_BGRAD_ATOMIC && opt->path == EP_PATH_UNFUSED)
    return fail(EP_ERR_UNSUPPORTED, "the unfused path uses the two-pass bias-gradient reduction only");
  return EP_OK;
}

GemmArgs base_args(const ep_shape* s, int cfg, bool dual) {
  GemmArgs a;
  memset(&a, 0, sizeof a);
  a.a = s->a;
  a.b = s->b;
  a.d = s->d;
  a.lda = s->lda;
  a.ldb = s->ldb;
  a.ldd = s->ldd;
  a.M = (int)s->m;
  a.N = (int)s->n;
  a.K = (int)s->k;
  const int bm = kTileCfgs[cfg].bm;
  const int bn = dual ? kTileCfgs[cfg].bnt / 2 : kTileCfgs[cfg].bnt;
  a.tiles_m = (int)((s->m + bm - 1) / bm);
  a.tiles_n = (int)((s->n + bn - 1) / bn);
  return a;
}

}  // namespace

extern "C" ep_status ep_plan_ex(const ep_shape* s, ep_dtype dtype, ep_epilog epi, const ep_epilog_io* io,
                                const ep_options* opt_in, ep_handle* out);
extern "C" ep_status ep_execute(ep_handle h, void* stream);
extern "C" ep_status ep_free(ep_handle h);

namespace {

// Plan-time tuning: every allowed (tile configuration, split) pair is planned, run once to
// warm up and three times under HIP events on the null stream, and the fastest is kept.
// The choice is cached for the process under the problem's key.
using TuneKey = std::tuple<int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int, int, int, int, int>;
std::mutex g_tune_mu;
struct TuneChoice {
  int cfg, split, tail;
};
std::map<TuneKey, TuneChoice> g_tune_cache;

ep_status autotune(const ep_shape* s, ep_dtype dtype, ep_epilog epi, const ep_epilog_io* io, ep_options& opt,
                   int dev) {
  const TuneKey key{s->m, s->n, s->k, s->lda, s->ldb, s->ldd, (int)s->b_layout + 2 * (int)s->a_layout,
                    (int)dtype, (int)epi, (int)opt.bgrad_mode, dev};
  {
    std::lock_guard<std::mutex> lk(g_tune_mu);
    auto it = g_tune_cache.find(key);
    if (it != g_tune_cache.end()) {
      opt.tile_cfg = it->second.cfg;
      opt.split_k = it->second.split;
      opt.split_tail = it->second.tail;
      opt.autotune = 0;
      return EP_OK;
    }
  }
  // Every candidate plan is built first and run once; then the candidates are timed in turn,
  // kRounds rounds of one execute each, so that clock and power drift during tuning affect
  // them alike; the median of each candidate's rounds decides.
  struct Cand {
    ep_handle h;
    int cfg, split, tail;
    std::vector<float> ms;
  };
  std::vector<Cand> cands;
  for (int c = 0; c < kNumTileCfgs; ++c) {
    for (int sp : {1, 0}) {  // unsplit, then the split the shape model picks (if it splits)
      ep_options o = opt;
      o.autotune = 0;
      o.tile_cfg = c;
      o.split_k = sp;
      ep_handle t = nullptr;
      if (ep_plan_ex(s, dtype, epi, io, &o, &t) != EP_OK) continue;
      if (sp == 0 && t->splits == 1) {  // the model does not split: same as the unsplit run
        ep_free(t);
        continue;
      }
      cands.push_back({t, c, t->splits, t->args.tail0 > 0 ? 1 : 0, {}});
    }
  }
  constexpr int kRounds = 5;
  // Before each timed execute a 512 MiB scratch buffer is overwritten (outside the events),
  // so that no candidate finds its operands in L2 or the Infinity Cache.  Without the buffer
  // (allocation failed) the candidates are timed warm.
  constexpr size_t kFlushBytes = size_t(512) << 20;
  void* flush = nullptr;
  if (hipMalloc(&flush, kFlushBytes) != hipSuccess) {
    flush = nullptr;
    (void)hipGetLastError();
  }
  hipEvent_t e0 = nullptr, e1 = nullptr;
  bool ok = hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess;
  for (auto& cd : cands) ok = ok && ep_execute(cd.h, nullptr) == EP_OK;
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  for (int r = 0; ok && r < kRounds; ++r) {
    for (auto& cd : cands) {
      float ms = 0.f;
      if (flush && hipMemsetAsync(flush, r, kFlushBytes, nullptr) != hipSuccess) ok = false;
      ok = ok && hipEventRecord(e0, nullptr) == hipSuccess && ep_execute(cd.h, nullptr) == EP_OK &&
           hipEventRecord(e1, nullptr) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
           hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
      if (!ok) break;
      cd.ms.push_back(ms);
    }
  }
  float best_ms = 1e30f;
  int best_cfg = -1, best_split = 1, best_tail = 0;
  for (auto& cd : cands) {
    if (ok && (int)cd.ms.size() == kRounds) {
      std::sort(cd.ms.begin(), cd.ms.end());
      const float med = cd.ms[kRounds / 2];
      if (med < best_ms) {
        best_ms = med;
        best_cfg = cd.cfg;
        best_split = cd.split;
        best_tail = cd.tail;
      }
    }
    ep_free(cd.h);
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (flush) (void)hipFree(flush);
  if (!ok) return fail(EP_ERR_HIP, "autotune: timing a candidate failed");
  if (best_cfg < 0) return fail(EP_ERR_INTERNAL, "autotune: no candidate configuration ran");
  {
    std::lock_guard<std::mutex> lk(g_tune_mu);
    g_tune_cache[key] = {best_cfg, best_split, best_tail};
  }
  t_last_error.clear();
  opt.tile_cfg = best_cfg;
  opt.split_k = best_split;
  opt.split_tail = best_tail;
  opt.autotune = 0;
  return EP_OK;
}

}  // namespace

namespace {

// What planning needs to know about a device, queried once per device (so that the
// allocation-free entry point makes no property query per call).
struct DevInfo {
  int cus;
  char arch[64];
};
constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
DevInfo g_dev[kMaxDevices];
bool g_dev_known[kMaxDevices];

ep_status device_info(int dev, DevInfo* out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(EP_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (!g_dev_known[dev]) {
      hipDeviceProp_t prop;
      hipError_t he = hipGetDeviceProperties(&prop, dev);
      if (he != hipSuccess) return fail(EP_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(he));
      g_dev[dev].cus = prop.multiProcessorCount;
      snprintf(g_dev[dev].arch, sizeof g_dev[dev].arch, "%s", prop.gcnArchName);
      g_dev_known[dev] = true;
    }
    *out = g_dev[dev];
  }
  if (strncmp(out->arch, "gfx950", 6) != 0)
    return fail(EP_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev, out->arch);
  return EP_OK;
}

// The device a stream launches on (the calling thread's current device for the null stream).
ep_status stream_device(hipStream_t s, int* dev) {
  if (s == nullptr) {
    if (hipGetDevice(dev) != hipSuccess) return fail(EP_ERR_HIP, "hipGetDevice failed");
    return EP_OK;
  }
  hipDevice_t sd = -1;
  if (hipStreamGetDevice(s, &sd) != hipSuccess) return fail(EP_ERR_INVALID_ARG, "the stream is not valid");
  *dev = (int)sd;
  return EP_OK;
}

size_t round_up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Plans into *h (value-initialised by the caller): tile configuration, split, kernels, kernel
// arguments and the workspace layout.  ws_limit is the most workspace the caller can provide: a
// split chosen by shape is reduced until its partials fit, and a plan that still needs more is
// EP_ERR_UNSUPPORTED.  Pointers into the workspace are set by bind_workspace.
ep_status plan_into(ep_plan_s* h, const ep_shape* s, ep_dtype dtype, ep_epilog epi, const ep_epilog_io* io,
                    const ep_options& opt, int dev, int cus, size_t ws_limit) {
  const bool dual = epi == EP_EPILOG_SWIGLU || epi == EP_EPILOG_SWIGLU_AUX;
  const bool unfused = opt.path == EP_PATH_UNFUSED;
  // the unfused path runs plain DEFAULT GEMMs (single-B) into intermediates
  const bool kernel_dual = dual && !unfused;
  if (opt.tile_cfg >= 0 && !cfg_allowed(opt.tile_cfg, kernel_dual, s->b_layout))
    return fail(EP_ERR_UNSUPPORTED, "tile_cfg %d cannot run SWIGLU with a K x N weight (needs a 256-row B tile)",
                opt.tile_cfg);
  if (opt.tile_cfg >= 0 && !cfg_fits_k(opt.tile_cfg, s->k))
    return fail(EP_ERR_UNSUPPORTED, "tile_cfg %d needs k to be a multiple of 64 (k = %lld)", opt.tile_cfg,
                (long long)s->k);
  const int cfg = opt.tile_cfg >= 0 ? opt.tile_cfg
                                    : pick_cfg(s, choose_cfg(s->m, s->n, kernel_dual, s->b_layout, cus), cus, kernel_dual);
  h->magic = kMagic;
  h->shape = *s;
  h->dtype = dtype;
  h->epilog = epi;
  h->io = *io;
  if (h->io.ld_aux == 0) h->io.ld_aux = (s->n + 31) / 32;
  if (h->io.ld_gu == 0) h->io.ld_gu = s->n;
  if (h->io.ldd2 == 0) h->io.ldd2 = epi == EP_EPILOG_SWIGLU_AUX ? 2 * s->n : s->ldd;
  if (h->io.ld_gelu_aux == 0) h->io.ld_gelu_aux = s->n;
  h->opt = opt;
  h->device = dev;
  h->cfg = cfg;

  GemmArgs a = base_args(s, cfg, kernel_dual);
  const int fused_epi = unfused ? (int)E_DEFAULT : (int)epi;
  const int klay = (int)s->b_layout + (s->a_layout == EP_A_KM ? 2 : 0);  // kernel layout index
  h->launch = gemm_launcher((int)dtype, klay, fused_epi, cfg);
  if (!h->launch) return fail(EP_ERR_INTERNAL, "no kernel instantiated for this combination");

  // ---- workspace pieces other than the split-K partials
  const int64_t M = s->m, N = s->n;
  const bool bgrad_epi = epi == EP_EPILOG_DRELU_BGRAD || epi == EP_EPILOG_DGELU_BGRAD;
  size_t part_bytes = 0, z_bytes = 0;
  if (bgrad_epi) {
    if (unfused) {
      // rows per column-sum block: about 1024 blocks of 2048 columns over the matrix, so
      // that every CU streams, within 32..256 rows (a multiple of 8)
      const int64_t col_blocks = (N + 2047) / 2048;
      int64_t rows = (M * col_blocks / 1024) / 8 * 8;
      rows = rows < 32 ? 32 : (rows > 256 ? 256 : rows);
      h->colsum_rows = (int)rows;
      h->nparts = (int)((M + h->colsum_rows - 1) / h->colsum_rows);
      part_bytes = (size_t)h->nparts * N * sizeof(float);
    } else if (opt.bgrad_mode == EP_BGRAD_TWO_PASS) {
      h->nparts = a.tiles_m;
      part_bytes = (size_t)h->nparts * N * sizeof(float);
    }
  }
  // the two branch GEMMs of the unfused SwiGLU need intermediates; every other unfused
  // sequence runs its elementwise passes in place on the output
  if (unfused && epi == EP_EPILOG_SWIGLU) z_bytes = (size_t)M * N * 2;

  // ---- split-K (fused path only)
  const int kt_all = (int)((s->k + kTileCfgs[cfg].bk - 1) / kTileCfgs[cfg].bk);
  const int64_t ntiles = (int64_t)a.tiles_m * a.tiles_n;
  const int slots = cus * kTileCfgs[cfg].occ;
  int tail0 = 0;  // tiles [0, tail0) run whole when a split plan splits only the last round's
  auto kpart_of = [&](int sp) {
    return sp > 1 ? (size_t)sp * (ntiles - tail0) * kTileCfgs[cfg].bm * kTileCfgs[cfg].bnt * sizeof(float) : 0;
  };
  auto total_of = [&](int sp) { return round_up256(part_bytes) + 2 * round_up256(z_bytes) + round_up256(kpart_of(sp)); };
  int splits = 1;
  if (!unfused) {
    if (opt.split_k > 0) {
      splits = opt.split_k;
      if (splits > 1 && opt.split_tail) {
        if (ntiles <= slots || ntiles % slots == 0)
          return fail(EP_ERR_UNSUPPORTED, "split_tail needs a partly filled last round (%lld tiles, %d slots)",
                      (long long)ntiles, slots);
        tail0 = (int)(ntiles / slots * slots);
      }
    } else {
      const SplitChoice c = choose_splits(ntiles, slots, kt_all, cfg);
      splits = c.splits;
      tail0 = c.tail0;
    }
    if (splits > kt_all) splits = kt_all;
    if (opt.split_k == 0)
      while (splits > 1 && total_of(splits) > ws_limit) --splits;
  }
  if (splits > 1) {
    a.kt_per_split = (kt_all + splits - 1) / splits;
    splits = (kt_all + a.kt_per_split - 1) / a.kt_per_split;  // no empty K range
  }
  if (splits == 1) tail0 = 0;
  h->splits = splits;
  a.splits = splits;
  a.tail0 = tail0;
  if (splits > 1) {
    h->launch_partial = gemm_partial_launcher((int)dtype, klay, kernel_dual, cfg);
    h->launch_fixup = gemm_fixup_launcher((int)dtype, (int)epi, cfg);
    if (!h->launch_partial || !h->launch_fixup)
      return fail(EP_ERR_INTERNAL, "no split-K kernel instantiated for this combination");
  }
  // one launch counts its work-items in 32 bits: the largest of the plan's GEMM grids (the
  // whole-K tiles, or every split range of the split tiles) must stay below 2^32 threads
  const int64_t blocks = splits > 1 ? std::max<int64_t>(tail0, (ntiles - tail0) * splits) : ntiles;
  if (blocks * kGemmWgThreads > (int64_t)UINT32_MAX)
    return fail(EP_ERR_UNSUPPORTED, "a grid of %lld workgroups of %lld threads exceeds one launch's 2^32 work-items",
                (long long)blocks, (long long)kGemmWgThreads);
  h->part_bytes = part_bytes;
  h->z_bytes = z_bytes;
  h->kpart_bytes = kpart_of(splits);
  h->workspace_bytes = total_of(splits);
  if (h->workspace_bytes > ws_limit)
    return fail(EP_ERR_UNSUPPORTED, "this plan needs %zu bytes of workspace; at most %zu are available",
                h->workspace_bytes, ws_limit);

  // ---- kernel arguments
  if (!unfused) {
    a.bias = io->bias;
    a.aux_out = io->relu_aux;
    a.aux_in = io->relu_aux_in;
    a.ld_aux = h->io.ld_aux;
    a.b2 = io->b2;
    a.gate = io->gate;
    a.up = io->up;
    a.ld_gu = h->io.ld_gu;
    a.d2 = io->d2;
    a.ldd2 = h->io.ldd2;
    a.gaux = io->gelu_aux;
    a.ld_gaux = h->io.ld_gelu_aux;
    if (bgrad_epi) {
      a.bgrad_atomic = opt.bgrad_mode == EP_BGRAD_ATOMIC;
      a.bgrad_part = a.bgrad_atomic ? io->bgrad : nullptr;  // two-pass: the partials (bind_workspace)
    }
    h->args = a;
  } else {
    // unfused: the GEMM writes its DEFAULT result straight to d (SWIGLU: to the two branch
    // intermediates; SWIGLU_AUX: to their halves of d2)
    if (epi == EP_EPILOG_SWIGLU) {
      a.d = nullptr;
      a.ldd = N;
    } else if (epi == EP_EPILOG_SWIGLU_AUX) {
      a.d = io->d2;
      a.ldd = h->io.ldd2;
    }
    h->args = a;
    if (dual) {
      GemmArgs a2 = a;
      a2.b = io->b2;
      a2.d = epi == EP_EPILOG_SWIGLU ? nullptr : (void*)((char*)io->d2 + N * 2);
      h->args2 = a2;
    }
  }
  if (getenv("EP_LOG")) {
    fprintf(stderr, "[ep] plan m=%lld n=%lld k=%lld %s %s %s cfg=%s tiles=%dx%d splits=%d ws=%zu\n", (long long)M,
            (long long)N, (long long)s->k, dtype == EP_F16 ? "f16" : "bf16", s->b_layout == EP_B_KN ? "KN" : "NK",
            kEpiNames[epi], kTileCfgs[cfg].name, a.tiles_m, a.tiles_n, splits, h->workspace_bytes);
    if (tail0 > 0) fprintf(stderr, "[ep]   split tail: tiles [0, %d) whole\n", tail0);
  }
  return EP_OK;
}

// Points every user of the workspace at its piece of ws (laid out as plan_into sized it).
void bind_workspace(ep_plan_s* h, void* ws) {
  char* w = (char*)ws;
  h->part = nullptr;
  h->uf.z = h->uf.z2 = nullptr;
  if (h->part_bytes) {
    h->part = (float*)w;
    w += round_up256(h->part_bytes);
  }
  if (h->z_bytes) {
    h->uf.z = w;
    w += round_up256(h->z_bytes);
    h->uf.z2 = w;
    w += round_up256(h->z_bytes);
  }
  h->args.part = h->kpart_bytes ? (float*)w : nullptr;
  h->uf.ldz = h->shape.n;
  const bool bgrad_epi = h->epilog == EP_EPILOG_DRELU_BGRAD || h->epilog == EP_EPILOG_DGELU_BGRAD;
  if (h->opt.path == EP_PATH_FUSED) {
    if (bgrad_epi && h->opt.bgrad_mode == EP_BGRAD_TWO_PASS) h->args.bgrad_part = h->part;
  } else if (h->epilog == EP_EPILOG_SWIGLU) {
    h->args.d = h->uf.z;
    h->args2.d = h->uf.z2;
  }
}

ep_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(EP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return EP_OK;
}

// status of a launch whose launcher returned the runtime's error itself
ep_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(EP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return EP_OK;
}

// Enqueues a bound plan's kernels on s.
ep_status launch_plan(const ep_plan_s* h, hipStream_t s) {
  const ep_shape& sh = h->shape;
  const int dt = (int)h->dtype;
  const int M = (int)sh.m, N = (int)sh.n;
  ep_status st;
  const bool bgrad_epi = h->epilog == EP_EPILOG_DRELU_BGRAD || h->epilog == EP_EPILOG_DGELU_BGRAD;
  if (h->opt.path == EP_PATH_FUSED) {
    if (bgrad_epi && h->opt.bgrad_mode == EP_BGRAD_ATOMIC) {
      if ((st = launched(launch_fill_zero_f32(h->io.bgrad, N, s), "fill_zero")) != EP_OK) return st;
    }
    if (h->splits > 1) {
      if (h->args.tail0 > 0) {  // the tiles of the whole rounds, then the split tail
        h->launch(h->args, s);
        if ((st = check_launch("fused gemm (whole rounds)")) != EP_OK) return st;
      }
      h->launch_partial(h->args, s);
      if ((st = check_launch("split-K partial gemm")) != EP_OK) return st;
      h->launch_fixup(h->args, s);
      if ((st = check_launch("split-K fixup + epilog")) != EP_OK) return st;
    } else {
      h->launch(h->args, s);
      if ((st = check_launch("fused gemm")) != EP_OK) return st;
    }
    if (bgrad_epi && h->opt.bgrad_mode == EP_BGRAD_TWO_PASS) {
      if ((st = launched(launch_bgrad_reduce(h->part, h->nparts, h->io.bgrad, N, s), "bgrad_reduce")) != EP_OK)
        return st;
    }
    return EP_OK;
  }
  // ---- unfused baseline: DEFAULT GEMM(s) then separate kernels through HBM, in place on d
  // (each launcher returns the launch's error: the status it took from the runtime is not
  // there for a later check_launch to see)
  h->launch(h->args, s);
  if ((st = check_launch("gemm")) != EP_OK) return st;
  switch (h->epilog) {
    case EP_EPILOG_DEFAULT:
      return EP_OK;
    case EP_EPILOG_BIAS:
      return launched(launch_bias_add(dt, sh.d, sh.ldd, h->io.bias, M, N, s), "bias_add");
    case EP_EPILOG_RELU_BIAS:
    case EP_EPILOG_RELU_AUX_BIAS:
      if ((st = launched(launch_bias_add(dt, sh.d, sh.ldd, h->io.bias, M, N, s), "bias_add")) != EP_OK) return st;
      return launched(launch_relu_pack(dt, sh.d, sh.ldd, sh.d, sh.ldd, h->io.relu_aux, h->io.ld_aux, M, N,
                                       h->epilog == EP_EPILOG_RELU_AUX_BIAS, s),
                      "relu_pack");
    case EP_EPILOG_DRELU_BGRAD:
      if ((st = launched(launch_mask_apply(dt, sh.d, sh.ldd, h->io.relu_aux_in, h->io.ld_aux, sh.d, sh.ldd, M, N, s),
                         "mask_apply")) != EP_OK)
        return st;
      if ((st = launched(launch_colsum_partial(dt, sh.d, sh.ldd, h->part, M, N, h->colsum_rows, s), "colsum")) != EP_OK)
        return st;
      return launched(launch_bgrad_reduce(h->part, h->nparts, h->io.bgrad, N, s), "bgrad_reduce");
    case EP_EPILOG_SWIGLU:
      h->launch(h->args2, s);
      if ((st = check_launch("gemm up")) != EP_OK) return st;
      return launched(launch_silu_mul(dt, h->uf.z, h->uf.z2, h->uf.ldz, sh.d, sh.ldd, M, N, s), "silu_mul");
    case EP_EPILOG_SWIGLU_AUX:
      h->launch(h->args2, s);
      if ((st = check_launch("gemm up")) != EP_OK) return st;
      return launched(launch_silu_mul(dt, h->io.d2, (const char*)h->io.d2 + N * 2, h->io.ldd2, sh.d, sh.ldd, M, N, s),
                      "silu_mul");
    case EP_EPILOG_DSWIGLU:
      return launched(launch_dswiglu(dt, sh.d, sh.ldd, h->io.gate, h->io.up, h->io.ld_gu, sh.d, sh.ldd, h->io.d2,
                                     h->io.ldd2, M, N, s),
                      "dswiglu");
    case EP_EPILOG_GELU_BIAS:
    case EP_EPILOG_GELU_AUX_BIAS:
      if ((st = launched(launch_bias_add(dt, sh.d, sh.ldd, h->io.bias, M, N, s), "bias_add")) != EP_OK) return st;
      return launched(launch_gelu_apply(dt, sh.d, sh.ldd, h->epilog == EP_EPILOG_GELU_AUX_BIAS ? h->io.gelu_aux : nullptr,
                                        h->io.ld_gelu_aux, M, N, s),
                      "gelu_apply");
    case EP_EPILOG_DGELU_BGRAD:
      if ((st = launched(launch_dgelu_apply(dt, sh.d, sh.ldd, h->io.gelu_aux, h->io.ld_gelu_aux, M, N, s),
                         "dgelu_apply")) != EP_OK)
        return st;
      if ((st = launched(launch_colsum_partial(dt, sh.d, sh.ldd, h->part, M, N, h->colsum_rows, s), "colsum")) != EP_OK)
        return st;
      return launched(launch_bgrad_reduce(h->part, h->nparts, h->io.bgrad, N, s), "bgrad_reduce");
  }
  return EP_OK;
}

// the plan's description, as ep_plan_info and ep_plan_describe write it
void describe(const ep_plan_s* h, char* buf, size_t n);

}  // namespace

extern "C" {

int ep_abi_version(void) { return EP_ABI_VERSION; }

int ep_num_tile_cfgs(void) { return kNumTileCfgs; }

const char* ep_status_string(ep_status s) {
  switch (s) {
    case EP_OK: return "EP_OK";
    case EP_ERR_INVALID_ARG: return "EP_ERR_INVALID_ARG";
    case EP_ERR_UNSUPPORTED: return "EP_ERR_UNSUPPORTED";
    case EP_ERR_OUT_OF_MEMORY: return "EP_ERR_OUT_OF_MEMORY";
    case EP_ERR_HIP: return "EP_ERR_HIP";
    case EP_ERR_INTERNAL: return "EP_ERR_INTERNAL";
  }
  return "EP_ERR_UNKNOWN";
}

const char* ep_last_error(void) { return t_last_error.c_str(); }

ep_status ep_plan(const ep_shape* shape, ep_dtype dtype, ep_epilog epilog, const ep_epilog_io* io, ep_handle* out) {
  return ep_plan_ex(shape, dtype, epilog, io, nullptr, out);
}

ep_status ep_plan_ex(const ep_shape* s, ep_dtype dtype, ep_epilog epi, const ep_epilog_io* io,
                     const ep_options* opt_in, ep_handle* out) {
  t_last_error.clear();
  if (!out) return fail(EP_ERR_INVALID_ARG, "out handle pointer is NULL");
  *out = nullptr;
  ep_status st = validate(s, dtype, epi, io, opt_in);
  if (st != EP_OK) return st;
  ep_options opt = opt_in ? *opt_in : ep_options{EP_PATH_FUSED, EP_BGRAD_TWO_PASS, -1, 0, 0};

  // ---- first HIP call: the device must exist and be usable
  int dev = -1;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return fail(EP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(he));
  DevInfo di;
  if ((st = device_info(dev, &di)) != EP_OK) return st;

  if (opt.autotune) {
    st = autotune(s, dtype, epi, io, opt, dev);
    if (st != EP_OK) return st;
  }

  ep_plan_s* h = new (std::nothrow) ep_plan_s{};  // every member zero / null
  if (!h) return fail(EP_ERR_OUT_OF_MEMORY, "host allocation failed");
  st = plan_into(h, s, dtype, epi, io, opt, dev, di.cus, SIZE_MAX);
  if (st != EP_OK) {
    delete h;
    return st;
  }
  if (h->workspace_bytes) {
    he = hipMalloc(&h->workspace, h->workspace_bytes);
    if (he != hipSuccess) {
      const size_t bytes = h->workspace_bytes;
      delete h;
      (void)hipGetLastError();
      return fail(EP_ERR_OUT_OF_MEMORY, "hipMalloc(%zu): %s", bytes, hipGetErrorString(he));
    }
  }
  bind_workspace(h, h->workspace);
  *out = h;
  return EP_OK;
}

ep_status ep_execute(ep_handle h, void* stream) {
  if (!h || h->magic != kMagic) return fail(EP_ERR_INVALID_ARG, "invalid or freed handle");
  hipStream_t s = (hipStream_t)stream;
  // The launches go to the stream's device (the calling thread's current device for the null
  // stream); the plan's pointers and workspace live on the device it was planned on.
  int dev = -1;
  ep_status st = stream_device(s, &dev);
  if (st != EP_OK) return st;
  if (dev != h->device)
    return fail(EP_ERR_INVALID_ARG, "the stream's device (%d) is not the device the plan was made on (%d)", dev,
                h->device);
  return launch_plan(h, s);
}

ep_status ep_execute_noalloc(const ep_shape* s, ep_dtype dtype, ep_epilog epi, const ep_epilog_io* io,
                             const ep_options* opt_in, void* stream) {
  t_last_error.clear();
  ep_status st = validate(s, dtype, epi, io, opt_in);
  if (st != EP_OK) return st;
  const ep_options opt = opt_in ? *opt_in : ep_options{EP_PATH_FUSED, EP_BGRAD_TWO_PASS, -1, 0, 0};
  if (opt.autotune) return fail(EP_ERR_INVALID_ARG, "autotune allocates its timing buffers; not available here");
  if (opt.path != EP_PATH_FUSED)
    return fail(EP_ERR_UNSUPPORTED, "the unfused path needs HBM intermediates; only the fused path runs here");
  int dev = -1;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return fail(EP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(he));
  hipStream_t hs = (hipStream_t)stream;
  int sdev = -1;
  if ((st = stream_device(hs, &sdev)) != EP_OK) return st;
  if (sdev != dev)
    return fail(EP_ERR_INVALID_ARG, "the stream's device (%d) is not the current device (%d)", sdev, dev);
  DevInfo di;
  if ((st = device_info(dev, &di)) != EP_OK) return st;
  void* scratch = nullptr;
  size_t cap = 0;
  he = static_scratch(dev, &scratch, &cap);
  if (he != hipSuccess) return fail(EP_ERR_HIP, "static scratch of device %d: %s", dev, hipGetErrorString(he));
  ep_plan_s h{};  // on the stack: nothing is allocated
  if ((st = plan_into(&h, s, dtype, epi, io, opt, dev, di.cus, cap)) != EP_OK) return st;
  bind_workspace(&h, scratch);
  return launch_plan(&h, hs);
}

ep_status ep_free(ep_handle h) {
  if (!h) return EP_OK;
  if (h->magic != kMagic) return fail(EP_ERR_INVALID_ARG, "invalid or already freed handle");
  h->magic = kDead;
  if (h->workspace) {
    hipError_t e = hipFree(h->workspace);
    h->workspace = nullptr;
    delete h;
    if (e != hipSuccess) return fail(EP_ERR_HIP, "hipFree: %s", hipGetErrorString(e));
    return EP_OK;
  }
  delete h;
  return EP_OK;
}

ep_status ep_plan_info(ep_handle h, char* buf, size_t n) {
  if (!h || h->magic != kMagic) return fail(EP_ERR_INVALID_ARG, "invalid or freed handle");
  if (!buf || n == 0) return fail(EP_ERR_INVALID_ARG, "buffer is NULL or empty");
  describe(h, buf, n);
  return EP_OK;
}

ep_status ep_plan_describe(const ep_shape* s, ep_dtype dtype, ep_epilog epi, const ep_epilog_io* io,
                           const ep_options* opt_in, int cus, char* buf, size_t n) {
  t_last_error.clear();
  if (!buf || n == 0) return fail(EP_ERR_INVALID_ARG, "buffer is NULL or empty");
  if (cus < 1 || cus > 65536) return fail(EP_ERR_INVALID_ARG, "cus %d is not in 1..65536", cus);
  ep_status st = validate(s, dtype, epi, io, opt_in);
  if (st != EP_OK) return st;
  const ep_options opt = opt_in ? *opt_in : ep_options{EP_PATH_FUSED, EP_BGRAD_TWO_PASS, -1, 0, 0};
  if (opt.autotune) return fail(EP_ERR_INVALID_ARG, "autotune times kernels on the device; not available here");
  ep_plan_s h{};  // planned on the stack, never bound to a workspace or launched
  if ((st = plan_into(&h, s, dtype, epi, io, opt, -1, cus, SIZE_MAX)) != EP_OK) return st;
  describe(&h, buf, n);
  return EP_OK;
}

}  // extern "C"

namespace {
void describe(const ep_plan_s* h, char* buf, size_t n) {
  const ep_shape& s = h->shape;
  const char* dt = h->dtype == EP_F16 ? "f16" : "bf16";
  const char* lay = s.a_layout == EP_A_KM ? (s.b_layout == EP_B_KN ? "A^T,KN" : "A^T,NK")
                                          : (s.b_layout == EP_B_KN ? "KN" : "NK");
  std::string kern = std::string("gemm_kernel<") + dt + "," + lay + "," +
                     (h->opt.path == EP_PATH_FUSED ? kEpiNames[h->epilog] : "DEFAULT") + "," +
                     kTileCfgs[h->cfg].name + ">";
  std::string extra;
  if (h->splits > 1) {
    if (h->args.tail0 > 0)
      kern += " on tiles [0, " + std::to_string(h->args.tail0) + "), split-K x" + std::to_string(h->splits) +
              " (partial + fixup) on the other " +
              std::to_string((int64_t)h->args.tiles_m * h->args.tiles_n - h->args.tail0);
    else
      kern += " split-K x" + std::to_string(h->splits) + " (partial + fixup)";
  }
  if (h->opt.path == EP_PATH_FUSED) {
    if (h->epilog == EP_EPILOG_DRELU_BGRAD || h->epilog == EP_EPILOG_DGELU_BGRAD)
      extra = h->opt.bgrad_mode == EP_BGRAD_TWO_PASS ? " + bgrad_reduce" : " (after fill_zero; atomic bgrad)";
  } else {
    switch (h->epilog) {
      case EP_EPILOG_BIAS: extra = " + bias_add"; break;
      case EP_EPILOG_RELU_BIAS: extra = " + bias_add + relu"; break;
      case EP_EPILOG_RELU_AUX_BIAS: extra = " + bias_add + relu_pack"; break;
      case EP_EPILOG_DRELU_BGRAD: extra = " + mask_apply + colsum + bgrad_reduce"; break;
      case EP_EPILOG_SWIGLU: extra = " x2 + silu_mul"; break;
      case EP_EPILOG_SWIGLU_AUX: extra = " x2 (into d2) + silu_mul"; break;
      case EP_EPILOG_DSWIGLU: extra = " + dswiglu"; break;
      case EP_EPILOG_GELU_BIAS: extra = " + bias_add + gelu"; break;
      case EP_EPILOG_GELU_AUX_BIAS: extra = " + bias_add + gelu (aux)"; break;
      case EP_EPILOG_DGELU_BGRAD: extra = " + dgelu_apply + colsum + bgrad_reduce"; break;
      default: break;
    }
  }
  snprintf(buf, n,
           "epilog=%s path=%s dtype=%s layout=%s m=%lld n=%lld k=%lld tile=%s tile_cfg=%d grid=%dx%d "
           "splits=%d split_tail0=%d workspace_bytes=%zu kernels=%s%s",
           kEpiNames[h->epilog], h->opt.path == EP_PATH_FUSED ? "fused" : "unfused", dt, lay, (long long)s.m,
           (long long)s.n, (long long)s.k, kTileCfgs[h->cfg].name, h->cfg, h->args.tiles_m, h->args.tiles_n,
           h->splits, h->args.tail0, h->workspace_bytes, kern.c_str(), extra.c_str());
}
}  // namespace
