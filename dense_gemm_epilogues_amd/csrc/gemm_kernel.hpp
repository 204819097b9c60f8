// Fused GEMM + epilogue kernel for CDNA4 (gfx950).
//
// One workgroup (4 wave64s in a 2x2 grid, one workgroup per CU) computes a BM x BN output
// tile with fp32 accumulators held in registers:
//   * A and B tiles of BK k-values move from global memory straight into LDS with 16-byte
//     buffer loads that write LDS (no register staging), through a ring of NST stages; the
//     loads of k-step kt + NST - 1 are spread evenly over k-step kt.  Hardware bounds checks
//     turn offsets past the matrix edges into zeros.
//   * k-contiguous tiles (A, and B given N x K) keep rows of BK elements with an XOR swizzle
//     of their 16-byte chunks, so the MFMA fragment reads are free of bank conflicts.  B given
//     K x N (N contiguous) is kept as [BK k][128 n] sub-tiles and read with the LDS transpose
//     read (ds_read_b64_tr_b16), which hands each lane the k-run of one column.
//   * The K loop issues v_mfma_f32_32x32x16_{f16,bf16} (lane l of a 32x32 block holds column
//     l%32 and rows 8*(r/4) + 4*(l/32) + r%4 of its 16 accumulator registers) or, in the m16
//     configurations, v_mfma_f32_16x16x32_{f16,bf16} (lane l of a 16x16 block holds column
//     l%16 and rows 4*(l/16) + r of its 4 registers; its operands are the 8 k-values
//     8*(l/16) .. +7 of row / column l%16).  Under sustained load the 16x16x32 form moves a
//     quarter of the accumulator data per instruction for half the FLOP, and the card, which
//     is limited by power there, sustains about 13% more FLOP/s with it.  The order of MFMAs,
//     fragment reads and loads inside a k-step is fixed explicitly, and the barrier between
//     k-steps waits only for the stage needed next.
//   * The epilogue runs on the fp32 accumulators: each wave stages a 32-row slab through
//     LDS so that every lane owns 8 consecutive columns of one row, applies the epilog
//     (bias, ReLU, mask packing, mask application + column sums, SiLU*mul, dSwiGLU) in
//     fp32 and writes each output once, with 16-byte row-contiguous stores.
//
// Epilogs follow "Fusing Matmul Epilogs with nvmath-python" (forward: RELU_BIAS,
// RELU_AUX_BIAS; backward: DRELU_BGRAD), the hotdry.top cuBLASLt post (BIAS, the
// plan/execute split) and gemm_swiglu_mlp_fusion.py (SwiGLU forward, dSwiGLU epilogue).
#pragma once
#include <type_traits>

#include "ep_internal.hpp"
#include "normal_dist.hpp"
#include "pair_sched.hpp"

namespace ep {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kMaxSplits = 8;  // split-K ranges per tile
constexpr int kGroupM = 8;
constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past every num_records we build

constexpr int cfg_bm(int cfg) { return kTileCfgs[cfg].bm; }
constexpr int cfg_bnt(int cfg) { return kTileCfgs[cfg].bnt; }
constexpr int cfg_bk(int cfg) { return kTileCfgs[cfg].bk; }
constexpr int cfg_nst(int cfg) { return kTileCfgs[cfg].nst; }
constexpr int cfg_occ(int cfg) { return kTileCfgs[cfg].occ; }
constexpr bool cfg_vst(int cfg) { return kTileCfgs[cfg].vst != 0; }
constexpr int cfg_mf(int cfg) { return kTileCfgs[cfg].mf; }
constexpr bool cfg_cfl(int cfg) { return kTileCfgs[cfg].cfl != 0; }
constexpr bool cfg_bar2(int cfg) { return kTileCfgs[cfg].bar2 != 0; }

// The 16x16x32 MFMAs are issued as inline asm whose accumulator operand must sit in AGPRs:
// with the builtin, the register allocator spreads the 64 four-register accumulators of a
// wave over both register files and copies them back and forth inside the K loop.  Inline
// asm hides the instruction from the compiler's hazard tracking, so a configuration using it
// must not spill or move registers around the MFMAs (the build's resource usage shows none
// for the one 16x16x32 configuration; a register-staged variant spilled and computed wrong
// sums).  Then the hazards are covered: an accumulator feeds the next MFMA on it a whole
// k-slice (64 MFMAs) later, explicit wait states separate the zeroed accumulators from the
// first MFMA and the last MFMA from the first reads of its results (mfma_drain), and
// fragments come from LDS reads, whose waits the compiler inserts for asm operands as for
// any other use.
template <int DT>
struct Elem;

template <>
struct Elem<T_F16> {
  static __device__ __forceinline__ float to_f32(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  }
  static __device__ __forceinline__ uint32_t from_f32(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
  }
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // 16x16x32 with the accumulator pinned to AGPRs (see mfma_acc below)
  static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    return c;
  }
};

template <>
struct Elem<T_BF16> {
  static __device__ __forceinline__ float to_f32(uint32_t bits) {
    return __builtin_bit_cast(float, bits << 16);
  }
  static __device__ __forceinline__ uint32_t from_f32(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
  }
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    return c;
  }
};

// Two floats to one word of two elements (lo in bits 0-15), rounded to nearest even: a
// two-element vector conversion, which gfx950 does in one v_cvt_pk_{f16,bf16}_f32.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == T_F16) {
    const f16x2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
}

template <int DT>
__device__ __forceinline__ u32x2 pack4(f32x4 v) {
  return u32x2{pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])};
}

template <int DT>
__device__ __forceinline__ u32x4 pack8(f32x4 a, f32x4 b) {
  const u32x2 x = pack4<DT>(a), y = pack4<DT>(b);
  return u32x4{x[0], x[1], y[0], y[1]};
}

template <int DT>
__device__ __forceinline__ f32x4 unpack4(u32x2 w) {
  using E = Elem<DT>;
  f32x4 v;
  v[0] = E::to_f32(w[0] & 0xffffu);
  v[1] = E::to_f32(w[0] >> 16);
  v[2] = E::to_f32(w[1] & 0xffffu);
  v[3] = E::to_f32(w[1] >> 16);
  return v;
}

// a & b in one v_and_b32 the compiler cannot see through (it would turn an AND with a
// sign-extended bit back into a compare and a select, two instructions and a hazard wait
// where a bit-field extract and this AND are two)
// Wait states between the last MFMA of the K loop and the first VALU / LDS read of its
// results: more than any MFMA form in this kernel needs (18 for a 16-pass result).
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

__device__ __forceinline__ uint32_t and_opaque(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Copy of one accumulator register for VALU use.  The operand constraint keeps the
// accumulators in AGPRs up to each use, so the epilogue copies them one at a time instead of
// moving all of them into VGPRs when the K loop ends.
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// Logistic function from its definition, 1 / (1 + e^-t), with e^-t = 2^(-t log2 e) on the
// hardware exp2.  t -> -inf gives 2^(+inf) = inf and 1/inf = 0; t -> +inf gives 1.
__device__ __forceinline__ float sigmoid_f(float t) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * t));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7fffffffLL ? 0x7fffffffu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// descriptor from an already clamped extent
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_raw(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// 32-bit LDS address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Workgroups are dispatched round-robin over the 8 XCDs, so workgroup bid runs on XCD bid % 8
// and the chip runs 256 of them at a time (one per CU).  When both tile counts are multiples of
// 16, each such round of 256 tiles is a 16 x 16 block of the output, and XCD x takes a 4 x 8
// sub-block of it: an XCD's L2 then fills 4 A and 8 B panels per round, and the whole chip
// touches 16 + 16 panels, which the 8 XCDs share through the Infinity Cache; successive rounds
// walk along the columns of a 16-row band, so the band's A panels stay cached.  (Each XCD working
// down its own rows, the chip touched 64 + 4 panels per round, too many to stay cached.)
// Otherwise each XCD gets a contiguous range of the tile order, walked in groups of kGroupM
// tile-rows, so that tiles sharing A rows / B columns share that XCD's L2.
__device__ __forceinline__ void map_tile(int bid, int nblocks, int tiles_m, int tiles_n, int& pm,
                                         int& pn) {
  // both orders are computed and one is selected (a branch here made the register allocator
  // spill the 64-deep 16x16 kernels)
  const int x = bid & 7, l = bid >> 3;
  const int rnd = l >> 5, j = l & 31;
  const int nbc = max(tiles_n >> 4, 1);
  const int br = rnd / nbc, bc = rnd - br * nbc;
  const int bm = br * 16 + 4 * (x >> 1) + (j & 3);
  const int bn = bc * 16 + 8 * (x & 1) + (j >> 2);
  const int q = nblocks >> 3, r = nblocks & 7;
  const int t = (x < r) ? x * (q + 1) + l : r * (q + 1) + (x - r) * q + l;
  const int group = kGroupM * tiles_n;
  const int g = t / group;
  const int first_m = g * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int w = t - g * group;
  const bool blk = ((tiles_m | tiles_n) & 15) == 0;
  pm = blk ? bm : first_m + w % gm;
  pn = blk ? bn : w / gm;
}

// XOR swizzle of the 16-byte chunks of an LDS tile row (CPR chunks per row): chunk c of row r
// is stored at chunk c ^ swf(r).  With this function the fragment reads (32 consecutive rows
// at one logical chunk per half-wave, ds_read_b128) run without LDS bank conflicts for both
// 64-byte and 128-byte rows on gfx950, as measured with SQ_LDS_BANK_CONFLICT; the variant
// ((r >> 1) ^ (r >> 3)) & 3 for 64-byte rows doubled the LDS cycles of every read.
template <int CPR>
__device__ __forceinline__ int swf(int r) {
  return (r ^ (r >> 3)) & (CPR - 1);
}

// LDS layouts of the 16x16x32 configurations (32-deep k-steps).  With the 32x32 layouts every
// 16x16 fragment read (16 rows at one chunk per 16-lane group) conflicts on two LDS banks
// (SQ_LDS_BANK_CONFLICT = half of the LDS cycles on MI355X).  A probe of the read pattern
// measured the same for every XOR swizzle of the chunks within a row, and none for:
//   * k-contiguous tiles, 64-byte rows, 1 KiB slots of 16 rows, configurations with cfl:
//     the 16-byte chunk c (k-values 8c .. 8c+7) of slot row r is stored in slot row r ^ 4c,
//     at chunk position r / 4; slot byte 16 L holds row 4 (L & 3) + (L >> 2 & 3), chunk
//     (L >> 4 ^ L) & 3.  Each DMA lane quad then reads 16 bytes of four rows.
//   * the same tiles without cfl: rows kept whole (each DMA lane quad reads one 64-byte row
//     piece) with the 32x32 chunk swizzle, and slot row 4i + j stored in slot row 4j + i.
//     Measured the faster of the two wherever B is given N x K (65536 x 16384 x 8192
//     backward 1173 -> 1213 TFLOP/s sustained, the down GEMM 0.396 -> 0.353 ms), 1-2 %
//     slower than spread chunks where only A is k-contiguous (B given K x N).
//   * [BK k][128 n] sub-tiles: as for 32x32 blocks (64-byte segment g of k-row k at segment
//     g ^ (k & 3)), and in addition the two 32-byte halves of each segment swap when bit 3 of
//     k is set, so that the lane groups reading k-rows 8 apart use opposite halves.
__device__ __forceinline__ int m16_slot_row(int lane) { return 4 * (lane & 3) + ((lane >> 2) & 3); }
// whole-row layout: slot row 4i + j stored in slot row 4j + i (its own inverse)
__device__ __forceinline__ int m16_row_perm(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int m16_slot_chunk(int lane) { return ((lane >> 4) ^ lane) & 3; }
__device__ __forceinline__ int m16_frag_addr(int r, int c) {  // byte offset of row r, chunk c
  return (((r & ~15) | ((r & 15) ^ (c << 2))) << 6) + (((r >> 2) & 3) << 4);
}
__device__ __forceinline__ int kn_col(int pch, int k, bool m16) {  // first column of 16-byte chunk pch
  const int piece = m16 ? ((pch & 3) ^ (((k >> 3) & 1) << 1)) : (pch & 3);
  return (((pch >> 2) ^ (k & 3)) << 5) + (piece << 3);
}

// k-contiguous tiles kept as whole rows (every configuration but the spread-chunk one): the LDS
// row holding tile row r, the tile row held in LDS row s, and the XOR applied to the 16-byte
// chunk index of row r.  32x32 blocks: rows in order, chunk swizzle swf.  16x16 blocks with
// 64-byte rows: slot rows transposed 4 x 4 (m16_row_perm, its own inverse), swizzle swf.
// 16x16 blocks with 128-byte rows (64-deep k-steps): see r128_*.
__device__ __forceinline__ int r128_row(int r);
__device__ __forceinline__ int r128_inv(int s);
__device__ __forceinline__ int r128_sig(int r);
template <int MF, int BK>
__device__ __forceinline__ int kc_row(int r) {
  if constexpr (MF == 32) return r;
  else if constexpr (BK == 32) return m16_row_perm(r);
  else return r128_row(r);
}
template <int MF, int BK>
__device__ __forceinline__ int kc_row_inv(int s) {
  if constexpr (MF == 32) return s;
  else if constexpr (BK == 32) return m16_row_perm(s);
  else return r128_inv(s);
}
template <int MF, int BK>
__device__ __forceinline__ int kc_sig(int r) {
  if constexpr (MF == 16 && BK == 64) return r128_sig(r);
  else return swf<BK / 8>(r);
}
// 128-byte rows read as 16x16 fragments (16 rows at one 16-byte chunk per 16-lane group): rows
// in order, chunk c of row r stored at chunk c ^ (r & 7).  A probe of exactly this read pattern
// over 24 layouts (row permutations within 8 and 16 rows x eight chunk swizzles) measured no
// bank conflict for it (SQ_LDS_BANK_CONFLICT 0, 4 LDS cycles per ds_read_b128, i.e. 256 bytes
// per clock), against conflicts on half or three quarters of the cycles for most others,
// swf's (r ^ r >> 3) & 7 included.  The DMA side is a whole row per 8 consecutive lanes.
__device__ __forceinline__ int r128_row(int r) { return r; }
__device__ __forceinline__ int r128_inv(int s) { return s; }
__device__ __forceinline__ int r128_sig(int r) { return r & 7; }

template <int DT, int LAY, int EPI, int CFG>
struct GemmTraits {
  static constexpr int BM = cfg_bm(CFG), BNT = cfg_bnt(CFG), BK = cfg_bk(CFG), NST = cfg_nst(CFG);
  static constexpr bool DUAL = EPI == E_SWIGLU || EPI == E_SWIGLU_AUX;
  static constexpr int WTM = BM / 2;             // rows per wave
  static constexpr int WTB = BNT / 2;            // B-tile rows per wave
  static constexpr int MF = cfg_mf(CFG);         // MFMA block edge (32 or 16)
  static constexpr int KMF = MF == 32 ? 16 : 32;  // k per MFMA
  static constexpr int ACC_R = MF * MF / 64;     // accumulator registers per block and lane
  static constexpr int MB = WTM / MF;            // MFMA blocks per wave along M
  static constexpr int NB = WTB / MF;            // ... along the B tile
  static constexpr int BN_OUT = DUAL ? BNT / 2 : BNT;
  static constexpr int WTN = DUAL ? WTB / 2 : WTB;  // output columns per wave
  static constexpr int KS = BK / KMF;            // MFMA k-slices per k-step
  static constexpr int ROWB = BK * 2;            // bytes per k-contiguous tile row
  static constexpr int CPR = BK / 8;             // 16-byte chunks per row
  static constexpr int A_BYTES = BM * ROWB;
  static constexpr int B_BYTES = BNT * ROWB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_SLOTS = A_BYTES / 1024 / 4;   // 1 KiB DMA slots per wave per stage
  static constexpr int B_SLOTS = B_BYTES / 1024 / 4;
  static constexpr int RPS = 1024 / ROWB;        // rows per DMA slot (k-contiguous tiles)
  static constexpr int KN_SUB = BK * 256;        // bytes of one [BK k][128 n] sub-tile
  static constexpr int KN_SPS = BK / 4;          // DMA slots per sub-tile
  // staging pitch in floats.  A staging write stores one float per lane: 32x32 blocks in 2
  // groups of 32 lanes 4 rows apart, 16x16 blocks in 4 groups of 16 lanes 4 rows apart.  With
  // 4 * pitch = 32 (mod 64) banks the 2 groups, with 4 * pitch = 16 (mod 64) the 4 groups,
  // fall on disjoint banks; the reads (16 bytes per lane, 8 lanes per row piece) are
  // conflict-free with either.  (Probed on MI355X with SQ_LDS_BANK_CONFLICT: the 16x16 writes
  // at pitch WTN + 8 conflicted on half of their LDS cycles, at WTN + 4 on none.)
  static constexpr int SPITCH = WTN + (MF == 16 ? 4 : 8);
  static constexpr int STG_FLOATS = 32 * SPITCH;  // per wave: one 32-row slab of the output
  static constexpr int BG_OFF = 4 * STG_FLOATS * 4;      // bytes; cross-wave bgrad exchange
  static constexpr int MASK_OFF = BG_OFF + 2 * WTN * 4;  // bytes; one slab's mask words per M-wave
  static constexpr int WPT = BN_OUT / 32;                  // mask words per tile row
  static constexpr int EPI_BYTES = MASK_OFF + 2 * 32 * WPT * 4;
  static constexpr int LDS_BYTES = (NST * STAGE > EPI_BYTES) ? NST * STAGE : EPI_BYTES;
  static constexpr int LPR = WTN / 8;            // lanes per staged row (8 columns each)
  static constexpr int RPI = 64 / LPR;           // staged rows per iteration
  static constexpr int ITERS = 32 / RPI;
  static_assert(LPR >= 4 && LPR <= 64, "staged rows must span whole lanes");
  static constexpr int NBO = DUAL ? NB / 2 : NB;  // accumulator blocks per output column range
  static constexpr int WPR = WTN / 32;            // mask words per wave row
  static_assert(DUAL || WPR == 2 || WPR == 4, "mask words per slab row must be 2 or 4");
  static_assert(!DUAL || NBO >= 1, "dual B needs a block per output column range");
  // staged rows per chunk of the store loop: 8 rows read together where the epilog is a plain
  // store; one row at a time where it has per-row inputs (measured faster on MI355X)
  // (RELU_AUX_BIAS with two workgroups per CU: 4 rows, whose mask bytes then fit the registers)
  static constexpr int CH = (EPI == E_DSWIGLU || EPI == E_DRELU_BGRAD || EPI == E_DGELU_BGRAD) ? 1
                            : (EPI == E_RELU_AUX_BIAS && cfg_occ(CFG) > 1)                     ? (ITERS < 4 ? ITERS : 4)
                                                                                                : (ITERS < 8 ? ITERS : 8);
  static_assert(KS == 1 || KS == 2 || KS == 4, "k-slices per step: 1, 2 or 4");
  static_assert(MF == 32 || MF == 16, "MFMA block edge");
  static_assert(MF == 32 || ((BK == 32 || (BK == 64 && NST == 2 && !cfg_cfl(CFG))) && !cfg_vst(CFG)),
                "16x16 LDS layouts: 32-deep k-steps, or 64-deep ones in a 2-stage ring, loaded directly");
  static_assert(MF == 16 || !cfg_cfl(CFG), "the conflict-free k-contiguous layout is for 16x16 blocks");
  static constexpr bool CFL = cfg_cfl(CFG);
  static_assert(A_SLOTS >= 1 && B_SLOTS >= 1, "tile too small for 1 KiB DMA slots");
  static_assert(LDS_BYTES * cfg_occ(CFG) <= 160 * 1024, "LDS budget");
};

// MODE 0: whole K range, then the epilog.  MODE 1 (split-K partial): of the nt = tiles -
// p.tail0 split tiles (tile indices before the XCD remap, from p.tail0 on), block b computes
// the K-steps [s * kt_per_split, (s + 1) * kt_per_split) of tile p.tail0 + b % nt, s = b / nt,
// and stores its fp32 accumulators to p.part.  MODE 2 (split-K fixup): block b sums the
// p.splits partials of tile p.tail0 + b in split order and runs the epilog (no K loop).  A
// split plan with p.tail0 > 0 runs tiles [0, p.tail0) whole in a MODE 0 launch of its own.
template <int DT, int LAY, int EPI, int CFG, int MODE>
__global__ __launch_bounds__(kThreads, cfg_occ(CFG)) void gemm_kernel(GemmArgs p) {
  using E = Elem<DT>;
  using TR = GemmTraits<DT, LAY, EPI, CFG>;
  // LAY: bit 0 = B layout (L_KN / L_NK); LAY >= 2: A is given K x M (M contiguous) and the
  // GEMM uses its transpose, staged like a K x N B operand
  constexpr int BLAY = LAY & 1;
  constexpr bool AKM = LAY >= 2;
  static_assert(!AKM || EPI == E_DEFAULT, "a K x M A operand is instantiated for DEFAULT only");
  constexpr bool DUAL = TR::DUAL;
  constexpr int BM = TR::BM, BNT = TR::BNT, BK = TR::BK, NST = TR::NST;
  constexpr int MB = TR::MB, NB = TR::NB, WTM = TR::WTM, WTB = TR::WTB, WTN = TR::WTN;
  constexpr int MF = TR::MF, KMF = TR::KMF, ACC_R = TR::ACC_R;
  using AccT = std::conditional_t<MF == 32, f32x16, f32x4>;
  constexpr int KS = TR::KS, ROWB = TR::ROWB, CPR = TR::CPR, RPS = TR::RPS;
  constexpr int A_SLOTS = TR::A_SLOTS, B_SLOTS = TR::B_SLOTS;

  __shared__ __attribute__((aligned(16))) char smem[TR::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wm = wave >> 1, wn = wave & 1;

  const int ntiles = p.tiles_m * p.tiles_n;
  const int nsplit = ntiles - p.tail0;  // tiles of the split range (MODE 1, 2)
  const int split = MODE == 1 ? (int)blockIdx.x / nsplit : 0;
  // tile index before the XCD remap
  const int tbid = MODE == 0 ? (int)blockIdx.x : p.tail0 + (int)blockIdx.x - split * nsplit;
  int pm, pn;
  map_tile(tbid, ntiles, p.tiles_m, p.tiles_n, pm, pn);
  const int m0 = pm * BM;
  const int n0 = pn * TR::BN_OUT;
  const int M = p.M, N = p.N, K = p.K;

  // DRELU_BGRAD: the mask words of the wave's 32-row slabs (32 rows x WPR words each), loaded
  // here so that their latency passes behind the K loop: word (row, w) of slab i sits in
  // register [i][row / RPW] of lane (row % RPW) * WPR + w
  constexpr int NSLAB = TR::WTM / 32;
  constexpr int WPR = TR::WPR;
  constexpr int NW = WPR / 2 > 0 ? WPR / 2 : 1;
  constexpr int RPW = 64 / WPR;
  uint32_t mw_all[EPI == E_DRELU_BGRAD ? NSLAB : 1][NW];
  if constexpr (EPI == E_DRELU_BGRAD && MODE != 1) {
#pragma unroll
    for (int i = 0; i < NSLAB; ++i)
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        const int grow = m0 + wm * TR::WTM + i * 32 + q * RPW + lane / WPR;
        const int wc = (n0 + wn * TR::WTN) / 32 + lane % WPR;
        mw_all[i][q] = (grow < M && wc * 32 < N) ? p.aux_in[(int64_t)grow * p.ld_aux + wc] : 0u;
      }
  }
  const int KT_ALL = (K + BK - 1) / BK;
  // this block's K-steps: [KT0, KTE); local k-step kt loads global k-step KT0 + kt, and every
  // k-step past KTE reads as zeros (its global index is replaced by KT_ALL, past K)
  const int KT0 = MODE == 1 ? split * p.kt_per_split : 0;
  const int KTE = MODE == 1 ? min(KT_ALL, KT0 + p.kt_per_split) : (MODE == 2 ? 0 : KT_ALL);
  const int KT = KTE > KT0 ? KTE - KT0 : 0;
  auto gkt = [&](int kt) { return KT0 + kt < KTE ? KT0 + kt : KT_ALL; };

  const char* Ag = (const char*)p.a;
  const char* Bg = (const char*)p.b;
  const char* B2g = DUAL ? (const char*)p.b2 : (const char*)p.b;

  // ---------------------------------------------------------------- loader setup
  // Tiles move HBM/L2 -> LDS with 16-byte buffer loads that write LDS directly (no VGPR
  // staging), NST stages deep.  One load per wave fills a contiguous 1 KiB LDS slot: lane L
  // writes bytes [16L, 16L+16) of the slot, so the swizzle is applied by choosing which
  // global chunk each lane fetches.  Out-of-range offsets (rows/columns past the matrix, the
  // k tail, k-steps past the end) read as zero and write zeros to LDS.
  // Buffer descriptors are built once per tile: A (and an N x K B) start at the tile's first
  // row, k = 0, and extend to the last row of the matrix, so rows past M (N) fall outside
  // num_records; the k offset of a k-step is added to the per-lane offset.  A K x N B is
  // re-based per k-step (its rows are k).
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(Ag + (int64_t)m0 * p.lda * 2, (int64_t)(M - m0) * p.lda * 2);
  uint32_t a_voff[A_SLOTS];
  int a_klim[A_SLOTS];  // the k-step offset k0 is valid for this lane iff k0 < klim
  // K x M A: BM/128 sub-tiles of [BK k][128 m]; each wave's slots lie in one sub-tile
  const int wa_mbase = ((wave * A_SLOTS) / TR::KN_SPS) * 128;
#pragma unroll
  for (int q = 0; q < A_SLOTS; ++q) {
    if constexpr (AKM) {
      const int t = (wave * A_SLOTS + q) % TR::KN_SPS;
      const int k = 4 * t + (lane >> 4);
      const int ml = kn_col(lane & 15, k, MF == 16);
      a_voff[q] = (m0 + wa_mbase + ml < M) ? (uint32_t)(k * p.lda * 2) + ml * 2 : kOOB;
      a_klim[q] = 0;
    } else {
      const int row = TR::CFL ? (wave * A_SLOTS + q) * RPS + m16_slot_row(lane)
                              : kc_row_inv<MF, BK>((wave * A_SLOTS + q) * RPS + lane / CPR);
      const int c = TR::CFL ? m16_slot_chunk(lane) : (lane % CPR) ^ kc_sig<MF, BK>(row);
      a_voff[q] = (uint32_t)(row * p.lda * 2) + c * 16;
      a_klim[q] = K - c * 8;
    }
  }
  // Each wave's B slots come from a single source: for N x K the wave loads BNT/4 rows
  // (DUAL: waves 0-1 the gate rows, waves 2-3 the up rows); for K x N the wave's slots lie in
  // one 128-column sub-tile.
  static_assert((B_SLOTS * 4) % 2 == 0, "B slots");
  const bool w_second = DUAL && wave >= 2;
  const int w_sub = (wave * B_SLOTS) / TR::KN_SPS;  // K x N sub-tile of this wave
  const int w_cbase = DUAL ? 0 : w_sub * 128;
  const char* w_bsrc = (DUAL && (BLAY == L_NK ? w_second : w_sub == 1)) ? B2g : Bg;
  const __amdgpu_buffer_rsrc_t rB_nk =
      make_rsrc(w_bsrc + (int64_t)n0 * p.ldb * 2, (int64_t)(N - n0) * p.ldb * 2);
  uint32_t b_voff[B_SLOTS];
  int b_klim[B_SLOTS];
#pragma unroll
  for (int q = 0; q < B_SLOTS; ++q) {
    const int s = wave * B_SLOTS + q;
    if constexpr (BLAY == L_NK) {
      const int row = TR::CFL ? s * RPS + m16_slot_row(lane) : kc_row_inv<MF, BK>(s * RPS + lane / CPR);
      const int c = TR::CFL ? m16_slot_chunk(lane) : (lane % CPR) ^ kc_sig<MF, BK>(row);
      const int srow = DUAL ? (row % (BNT / 2)) : row;
      b_voff[q] = (uint32_t)(srow * p.ldb * 2) + c * 16;
      b_klim[q] = K - c * 8;
    } else {
      // B tile = BNT/128 sub-tiles of [BK k][128 n] (256-byte rows); 64-byte segment g of
      // k-row k is stored at segment g ^ (k & 3) (see kn_col).  DUAL: sub-tile 0 = gate,
      // 1 = up columns.
      const int t = s % TR::KN_SPS;
      const int k = 4 * t + (lane >> 4);
      const int nl = kn_col(lane & 15, k, MF == 16);
      // relative to the sub-tile's column base; columns past N read as zero
      b_voff[q] = (n0 + w_cbase + nl < N) ? (uint32_t)(k * p.ldb * 2) + nl * 2 : kOOB;
      b_klim[q] = 0;
    }
  }
  // K x N: base and clamped extent of this wave's sub-tile for the k-step being loaded
  // (descriptor values are not passed between functions: the host pass cannot take them)
  struct KnSrc {
    const char* base;   // K x N B: this wave's sub-tile for the k-step
    uint32_t num;
    const char* abase;  // K x M A: the same for A
    uint32_t anum;
  };
  auto kn_rsrc = [&](int kt) __attribute__((always_inline)) {
    const int k0 = gkt(kt) * BK;
    KnSrc s;
    const int64_t bytes = ((int64_t)(K - k0) * p.ldb - (n0 + w_cbase)) * 2;
    s.base = w_bsrc + ((int64_t)k0 * p.ldb + n0 + w_cbase) * 2;
    s.num = bytes <= 0 ? 0u : (bytes >= 0x7fffffffLL ? 0x7fffffffu : (uint32_t)bytes);
    s.abase = Ag;
    s.anum = 0u;
    if constexpr (AKM) {
      const int64_t abytes = ((int64_t)(K - k0) * p.lda - (m0 + wa_mbase)) * 2;
      s.abase = Ag + ((int64_t)k0 * p.lda + m0 + wa_mbase) * 2;
      s.anum = abytes <= 0 ? 0u : (abytes >= 0x7fffffffLL ? 0x7fffffffu : (uint32_t)abytes);
    }
    return s;
  };

  // One DMA op = one 1 KiB slot of a stage (A slots first, then B slots).
  constexpr int N_DMA = A_SLOTS + B_SLOTS;
  // The 64-deep 16x16 configuration runs only with K a multiple of 64 (the planner's rule), so
  // each k-contiguous load lies wholly inside K: its k offset goes in the instruction's scalar
  // offset and the per-lane offset is fixed for the tile (it still range-checks the rows: rows
  // past the matrix read zeros).  A k-step past the block's range reloads the last k-step of the
  // matrix instead of reading zeros: its stage is never read.  The other configurations compare
  // each lane's chunk with K per load (chunks past K and k-steps past the end read zeros).
  constexpr bool SOFF = MF == 16 && BK == 64 && NST == 2;
  auto dma_op = [&](int kt, char* As, int t, const KnSrc& kr, auto full_c) __attribute__((always_inline)) {
    const int k0 = gkt(kt) * BK;
    constexpr bool kfull = SOFF;
    (void)full_c;
    const int ksoff = (gkt(kt) < KT_ALL ? gkt(kt) : KT_ALL - 1) * BK * 2;  // kfull: scalar k offset in bytes
    if (t < A_SLOTS) {
      const int q = t;
      if constexpr (AKM) {
        const __amdgpu_buffer_rsrc_t rka = make_rsrc_raw(kr.abase, kr.anum);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rka, (__attribute__((address_space(3))) void*)(As + (wave * A_SLOTS + q) * 1024), 16, (int)a_voff[q], 0, 0, 0);
      } else if constexpr (kfull) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rA, (__attribute__((address_space(3))) void*)(As + (wave * A_SLOTS + q) * 1024), 16, (int)a_voff[q], ksoff, 0, 0);
      } else {
        const uint32_t off = (k0 < a_klim[q]) ? a_voff[q] + k0 * 2 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rA, (__attribute__((address_space(3))) void*)(As + (wave * A_SLOTS + q) * 1024), 16, (int)off, 0, 0, 0);
      }
    } else {
      const int q = t - A_SLOTS;
      char* Bs = As + TR::A_BYTES;
      if constexpr (BLAY == L_NK) {
        if constexpr (kfull) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rB_nk, (__attribute__((address_space(3))) void*)(Bs + (wave * B_SLOTS + q) * 1024), 16, (int)b_voff[q], ksoff, 0, 0);
        } else {
          const uint32_t off = (k0 < b_klim[q]) ? b_voff[q] + k0 * 2 : kOOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rB_nk, (__attribute__((address_space(3))) void*)(Bs + (wave * B_SLOTS + q) * 1024), 16, (int)off, 0, 0, 0);
        }
      } else {
        const __amdgpu_buffer_rsrc_t rk = make_rsrc_raw(kr.base, kr.num);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (__attribute__((address_space(3))) void*)(Bs + (wave * B_SLOTS + q) * 1024), 16, (int)b_voff[q], 0, 0, 0);
      }
    }
  };
  auto issue_tile = [&](int kt, char* As) __attribute__((always_inline)) {
    const KnSrc kr = kn_rsrc(kt);
#pragma unroll
    for (int t = 0; t < N_DMA; ++t) dma_op(kt, As, t, kr, std::false_type{});
  };

  // Register staging (vst configurations): the same 16 bytes per lane as dma_op, loaded into
  // registers (sreg[t]) one k-step ahead and written to the lane's 16 bytes of the slot later.
  constexpr bool VST = cfg_vst(CFG);
  static_assert(!VST || NST == 2, "register staging feeds a 2-stage LDS ring");
  u32x4 sreg[VST ? N_DMA : 1];
  auto gload = [&](int kt, int t, const KnSrc& kr) __attribute__((always_inline)) -> u32x4 {
    const int k0 = gkt(kt) * BK;
    if (t < A_SLOTS) {
      const int q = t;
      if constexpr (AKM) {
        return __builtin_amdgcn_raw_buffer_load_b128(make_rsrc_raw(kr.abase, kr.anum), (int)a_voff[q], 0, 0);
      } else {
        const uint32_t off = (k0 < a_klim[q]) ? a_voff[q] + k0 * 2 : kOOB;
        return __builtin_amdgcn_raw_buffer_load_b128(rA, (int)off, 0, 0);
      }
    } else {
      const int q = t - A_SLOTS;
      if constexpr (BLAY == L_NK) {
        const uint32_t off = (k0 < b_klim[q]) ? b_voff[q] + k0 * 2 : kOOB;
        return __builtin_amdgcn_raw_buffer_load_b128(rB_nk, (int)off, 0, 0);
      } else {
        return __builtin_amdgcn_raw_buffer_load_b128(make_rsrc_raw(kr.base, kr.num), (int)b_voff[q], 0, 0);
      }
    }
  };
  auto lput = [&](char* As, int t) __attribute__((always_inline)) {
    char* slot = t < A_SLOTS ? As + (wave * A_SLOTS + t) * 1024
                             : As + TR::A_BYTES + (wave * B_SLOTS + (t - A_SLOTS)) * 1024;
    *(u32x4*)(slot + lane * 16) = sreg[t];
  };

  // fragment-read addresses
  const int hlf = lane >> 5;
  // the lane's 8-element k-chunk within a k-slice: 32x32x16 takes k 8*(l/32) .. +7 of 16,
  // 16x16x32 k 8*(l/16) .. +7 of 32; CPS 16-byte chunks per k-slice
  const int kq = MF == 32 ? hlf : (lane >> 4);
  constexpr int CPS = KMF / 8;
  uint32_t a_rd[MB], b_rd[NB];
  int a_f[MB], b_f[NB];
  // transpose-read address of an MF-wide block at column (row) base `base` of a [BK][128]
  // sub-tile layout: within each 16-lane group g, lane i fetches 4 columns of k-row
  // kbase + i/4; the hardware hands lane i the 4 k-values of column i.  32-wide blocks:
  // groups 0-1 read k 0-7, groups 2-3 k 8-15, odd groups the block's columns 16-31;
  // 16-wide blocks: group g reads k 8g .. 8g+7 of the block's 16 columns.
  auto tr_addr = [&](int base) __attribute__((always_inline)) {
    const int g = lane >> 4, i = lane & 15;
    const int u = base >> 7, cb = base & 127;
    const int krow = MF == 32 ? 8 * (g >> 1) + (i >> 2) : 8 * g + (i >> 2);
    const int cbyte = MF == 32 ? 32 * (g & 1) : 32 * (((cb & 31) >> 4) ^ ((krow >> 3) & 1));
    return (uint32_t)(u * TR::KN_SUB + krow * 256 + ((((cb >> 5) ^ (i >> 2)) & 3) << 6) + cbyte + 8 * (i & 3));
  };
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    if constexpr (AKM) {
      a_rd[i] = tr_addr(wm * WTM + i * MF);
      a_f[i] = 0;
    } else if constexpr (TR::CFL) {
      a_rd[i] = m16_frag_addr(wm * WTM + i * MF + (lane & 15), kq);
      a_f[i] = 0;
    } else {
      const int row = wm * WTM + i * MF + (lane & (MF - 1));
      a_rd[i] = kc_row<MF, BK>(row) * ROWB;
      a_f[i] = kc_sig<MF, BK>(row);
    }
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    int brow;
    if constexpr (DUAL) {
      brow = (j < NB / 2) ? wn * (WTB / 2) + j * MF : BNT / 2 + wn * (WTB / 2) + (j - NB / 2) * MF;
    } else {
      brow = wn * WTB + j * MF;
    }
    if constexpr (BLAY == L_NK && TR::CFL) {
      b_rd[j] = m16_frag_addr(brow + (lane & 15), kq);
      b_f[j] = 0;
    } else if constexpr (BLAY == L_NK) {
      const int row = brow + (lane & (MF - 1));
      b_rd[j] = kc_row<MF, BK>(row) * ROWB;
      b_f[j] = kc_sig<MF, BK>(row);
    } else {
      b_rd[j] = tr_addr(brow);
      b_f[j] = 0;
    }
  }

  AccT acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < ACC_R; ++r) acc[i][j][r] = 0.0f;
  if constexpr (MF == 16) {
    // the zeros are in the AGPRs, with wait states after them, before the first asm MFMA
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) asm volatile("" : "+a"(acc[i][j]));
    mfma_drain();
  }

  // ---------------------------------------------------------------- main loop
  u32x4 fa[2][MB], fb[2][NB];
  // One read op = one LDS fragment read: A blocks first, then B blocks (K x N: two
  // transpose reads of 4 k-values each per block).
  constexpr int A_OPS = AKM ? 2 * MB : MB;
  constexpr int B_OPS = (BLAY == L_NK) ? NB : 2 * NB;
  constexpr int N_RD = A_OPS + B_OPS;
  // Transpose reads are issued as inline asm: the compiler's LDS-DMA alias check would
  // otherwise make every one wait for all in-flight loads of later stages (which never
  // alias the stage being read).  Completion is awaited explicitly (lgkm_fence) before use.
  auto tr_read = [&](uint32_t addr, u32x4& dst, int half) __attribute__((always_inline)) {
    u32x2 w;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(w) : "v"(addr));
    dst[2 * half] = w[0];
    dst[2 * half + 1] = w[1];
  };
  // (a k-slice of a [BK][128] sub-tile is KMF k-rows of 256 bytes; the second transpose
  // read of a fragment is 4 k-rows further)
  auto read_op = [&](const char* As, int ks, int r, u32x4* A, u32x4* B) __attribute__((always_inline)) {
    if (r < A_OPS) {
      if constexpr (AKM) {
        const int i = r >> 1, half = r & 1;
        tr_read(lds_addr(As + a_rd[i]) + ks * KMF * 256 + half * 1024, A[i], half);
      } else if constexpr (TR::CFL) {
        A[r] = *(const u32x4*)(As + a_rd[r]);  // (one k-slice per k-step)
      } else {
        A[r] = *(const u32x4*)(As + a_rd[r] + ((((ks * CPS + kq) ^ a_f[r]) & (CPR - 1)) << 4));
      }
      return;
    }
    const char* Bs = As + TR::A_BYTES;
    if constexpr (BLAY == L_NK && TR::CFL) {
      B[r - A_OPS] = *(const u32x4*)(Bs + b_rd[r - A_OPS]);
    } else if constexpr (BLAY == L_NK) {
      const int j = r - A_OPS;
      B[j] = *(const u32x4*)(Bs + b_rd[j] + ((((ks * CPS + kq) ^ b_f[j]) & (CPR - 1)) << 4));
    } else {
      const int j = (r - A_OPS) >> 1, half = (r - A_OPS) & 1;
      tr_read(lds_addr(Bs + b_rd[j]) + ks * KMF * 256 + half * 1024, B[j], half);
    }
  };
  auto read_frags = [&](const char* As, int ks, u32x4* A, u32x4* B) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < N_RD; ++r) read_op(As, ks, r, A, B);
  };
  // Wait for every outstanding LDS read and tie the wait to the fragments the transpose
  // reads wrote, so no MFMA that consumes them can be scheduled above it.
  auto tie4 = [&](u32x4* F, auto n_c) __attribute__((always_inline)) {
    constexpr int NF = decltype(n_c)::value;
    static_assert(NF == 1 || NF == 2 || NF == 4 || NF == 8, "unsupported fragment count");
    if constexpr (NF == 8) {
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(F[0]), "+v"(F[1]), "+v"(F[2]), "+v"(F[3]), "+v"(F[4]), "+v"(F[5]), "+v"(F[6]), "+v"(F[7]));
    } else if constexpr (NF == 4) {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(F[0]), "+v"(F[1]), "+v"(F[2]), "+v"(F[3]));
    } else if constexpr (NF == 2) {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(F[0]), "+v"(F[1]));
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(F[0]));
    }
  };
  auto lgkm_fence = [&](u32x4* A, u32x4* B) __attribute__((always_inline)) {
    if constexpr (AKM) tie4(A, std::integral_constant<int, MB>{});
    if constexpr (BLAY == L_KN) tie4(B, std::integral_constant<int, NB>{});
  };
  // The instruction order inside a k-step is fixed explicitly: every sched_barrier below
  // stops the scheduler from moving instructions across it.  Each MFMA is followed by its
  // share of the fragment reads of the next k-slice, and the DMA loads of the stage NST-1
  // k-steps ahead are spread evenly over the whole k-step (one every DSTRIDE MFMAs): issued
  // in bursts they fill the texture-address FIFO and stall the MFMA stream behind them.
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  constexpr int NMMA = MB * NB;
  constexpr int TOT = KS * NMMA;                       // MFMAs per k-step
  // With only 2 stages the loads of the next stage must land before this k-step's barrier,
  // so they are issued in the first half of the k-step; with more stages, over all of it.
  // Register staging writes the next stage from registers, which must happen before the
  // barrier (GBAR below): spread over the first three quarters (measured 1-2.5 % faster than
  // the first half, whose LDS writes crowd the fragment reads).
  // Two barriers per k-step (16x16 blocks, 64-deep k-steps in a 2-stage ring).  The first, at
  // MFMA POST_BA, follows the reads of the k-step's second-slice fragments: every wave is then
  // done with stage kt % 2, and the loads of k-step kt + 2 go into it, spread evenly up to the
  // second barrier, HB MFMAs into the second slice.  The second barrier waits for the loads of
  // k-step kt + 1 (issued a k-step earlier; this k-step's own loads may stay in flight) before
  // the next k-step's first-slice fragments are read from its stage.  A load thus has from its
  // issue to the next k-step's second barrier -- a k-step or more -- to land.  Each 128-byte row
  // piece is a whole cache line fetched by 8 consecutive lanes.  (POST_BA 0: one barrier, between
  // the slices, with the loads after it.)
  constexpr bool POSTW = MF == 16 && NST == 2 && !VST;
  // (two barriers measured 2.7 % faster where both operands are k-contiguous -- B given N x K.
  // Where B is given K x N they are 2-7 % faster on the shorter K loops -- the K-concatenated
  // 2048 x 5120 x 34816 dx GEMM split 3 ways 0.627 -> 0.590 ms, 2048 x 17408 x 5120 0.314 ->
  // 0.305 ms, its dSwiGLU form 0.378 -> 0.352 ms, 16384 x 17408 x 5120 2.048 -> 2.005 ms -- but
  // 0.5-1 % slower on the 65536 x 8192 x 16384 forward: configuration 12 has them for K x N B
  // too, configuration 11 only for N x K.)
  constexpr int POST_BA = (POSTW && !AKM && (BLAY == L_NK || cfg_bar2(CFG))) ? 20 : 0;
  constexpr int HB = POSTW ? (POST_BA > 0 ? NMMA / 2 : 0) : (NMMA >= 8 ? NMMA / 4 : NMMA / 2);  // MFMAs of the last slice before the barrier
  // DMA ops of the current k-step issued before its barrier
  constexpr int GBAR = (KS - 1) * NMMA + HB;
  constexpr int DWIN = VST ? ((TOT * 3) / 4 < GBAR ? (TOT * 3) / 4 : GBAR) : (NST == 2 ? TOT / 2 : TOT);
  constexpr int DSTRIDE = DWIN / N_DMA > 0 ? DWIN / N_DMA : 1;
  constexpr int DPER = (N_DMA + DWIN - 1) / DWIN;      // DMA ops per issue point
  // two-barrier k-steps: the MFMA window the loads are spread over
  constexpr int POST_LW0 = POST_BA > 0 ? POST_BA : GBAR;
  constexpr int POST_LW1 = POST_BA > 0 ? GBAR : TOT;
  static_assert(!POSTW || (KS == 2 && POST_LW1 - POST_LW0 >= N_DMA && POST_BA < NMMA), "post-barrier load window");
  // K-step pairs (16x16 configurations with A given M x K).  A k-contiguous operand arrives
  // as row pieces of 64 bytes per k-step: half of a 128-byte cache line, whose other half the
  // next k-step loads.  Loaded one k-step at a time, every line is fetched from L2 twice (the
  // L1 has long evicted it by then).  Here k-steps kt+3 and kt+4 (kt odd) are loaded
  // together, slot by slot alternately, so that the second load of a line meets the first
  // one's fill in the L1: L2 read requests halve (TCP_TCC_READ_REQ).  Paired are all slots
  // when B is N x K (configuration 10), A's when B is K x N (its rows are whole lines; B is
  // loaded every k-step as before).  Stage (kt+4) % NST is the one k-step kt consumes, free
  // once the k-step's barrier has passed, so the pair's loads start there and run into the
  // next k-step (pair_sched).
  constexpr bool PAIR = MF == 16 && NST == 4 && !VST && KS == 1 && !AKM && (BLAY == L_KN || !TR::CFL);
  constexpr int NPS = BLAY == L_NK ? N_DMA : A_SLOTS, NU = N_DMA - NPS;  // paired, unpaired slots
  constexpr PairSched PS_ = PAIR ? pair_sched(NMMA, HB, NPS, NU, N_DMA) : PairSched{2, 1, 1, 1, 0, 0, 0};
  static_assert(!PAIR || (PS_.ps >= 2 && HB % PS_.ps == 0 && (NMMA - HB) % PS_.ps == 0 && PS_.pafter < 2 * NPS &&
                          (NU == 0 || (NMMA % NU == 0 && PS_.us % PS_.ps == 0))), "pair load schedule");
  static_assert(!PAIR || (PS_.vmc_odd <= 63 && PS_.vmc_even <= 63 && PS_.vmc_pro <= 63), "vmcnt range");
  // odd k-step kt: stage of k-step kt+4; even kt: of k-step kt+2 (the pair begun in kt-1)
  char* pair_dst = smem;
  auto slice = [&](auto rd_c, auto g0_c, const u32x4* A, const u32x4* B, auto t0_c, auto t1_c, int kt,
                   char* dst, const KnSrc& kr, const char* rstage, int rks, u32x4* RA, u32x4* RB, auto par_s,
                   auto full_c) __attribute__((always_inline)) {
    constexpr bool RD = decltype(rd_c)::value;
    constexpr int G0 = decltype(g0_c)::value;        // k-step MFMA index of MFMA t = 0
    constexpr int T0 = decltype(t0_c)::value, T1 = decltype(t1_c)::value;
    // fragment reads per MFMA so that they finish (when the slice is long enough) 4 MFMAs
    // before the end of the slice
    // (16x16 blocks: 12 MFMAs before the end, as the MFMAs are half as long; the k-step's
    // first MFMA then finds its fragments landed)
    constexpr int RTAIL = MF == 16 ? 12 : 4;
    constexpr int RSPAN = (T1 - T0) > 2 * RTAIL ? (T1 - T0) - RTAIL : ((T1 - T0) > 8 ? (T1 - T0) - 4 : (T1 - T0));
    constexpr int RPM = RSPAN > 0 ? (N_RD + RSPAN - 1) / RSPAN : 1;
#pragma unroll
    for (int t = T0; t < T1; ++t) {
      acc[t / NB][t % NB] = E::mfma(A[t / NB], B[t % NB], acc[t / NB][t % NB]);
      const int g = G0 + t;
      if constexpr (PAIR) {
        // load d of a pair: slot d / 2 (paired slots come first: all, or A's) of its first
        // (d even) or second k-step.  The slice gets kt = k-step + 3, its stage and its K x N
        // source, which only the unpaired (K x N B) slots use.
        constexpr int PS = PS_.ps, PAFTER = PS_.pafter;
        if (decltype(par_s)::value == 1 && g >= HB && (g - HB) % PS == 0) {
          const int d = (g - HB) / PS;  // pair (kt, kt + 1), this k-step's loads 0 .. PAFTER-1
          if (d & 1)
            dma_op(kt + 1, pair_dst, d >> 1, kr, std::false_type{});
          else
            dma_op(kt, dst, d >> 1, kr, std::false_type{});
        } else if (decltype(par_s)::value == 0 && g < HB && g % PS == 0) {
          const int d = PAFTER + g / PS;  // pair (kt - 1, kt), its loads PAFTER .. 2 NPS-1
          if (d & 1)
            dma_op(kt, dst, d >> 1, kr, std::false_type{});
          else
            dma_op(kt - 1, pair_dst, d >> 1, kr, std::false_type{});
        }
        if constexpr (NU > 0) {
          if (g % PS_.us == PS_.uoff) dma_op(kt, dst, NPS + g / PS_.us, kr, std::false_type{});
        }
      } else if constexpr (POSTW) {
        // load d at MFMA POST_LW0 + floor(d * window / N_DMA): g issues load ceil((g - LW0) N_DMA / window)
        // when that load's position is g
        constexpr int WIN = POST_LW1 - POST_LW0;
        const int d = ((g - POST_LW0) * N_DMA + WIN - 1) / WIN;
        if (g >= POST_LW0 && d < N_DMA && POST_LW0 + (d * WIN) / N_DMA == g) dma_op(kt, dst, d, kr, full_c);
      } else if (g % DSTRIDE == 0) {
#pragma unroll
        for (int d = (g / DSTRIDE) * DPER; d < (g / DSTRIDE + 1) * DPER; ++d)
          if (d < N_DMA) {
            if constexpr (VST) {
              lput(dst, d);              // k-step kt - 1 (loaded one k-step ago) into its stage
              sreg[d] = gload(kt, d, kr);  // k-step kt into the freed register
            } else {
              dma_op(kt, dst, d, kr, std::false_type{});
            }
          }
      }
      if constexpr (RD) {
#pragma unroll
        for (int r = (t - T0) * RPM; r < (t - T0 + 1) * RPM; ++r)
          if (r < N_RD) read_op(rstage, rks, r, RA, RB);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using Z_ = std::integral_constant<int, 0>;
  using H_ = std::integral_constant<int, HB>;
  using W_ = std::integral_constant<int, NMMA>;
  static_assert(!VST || DWIN <= GBAR, "register-staged writes must precede the k-step barrier");
  constexpr int DPRE_RAW = ((GBAR + DSTRIDE - 1) / DSTRIDE) * DPER;
  constexpr int DPRE = DPRE_RAW < N_DMA ? DPRE_RAW : N_DMA;
  // Workgroup barrier that does not drain the DMA ring: wait until this wave's loads of the
  // stage needed next (k-step kt+1) have landed -- everything younger may stay in flight --
  // and for its LDS reads, then s_barrier.  The memory clobber keeps the compiler from
  // moving LDS accesses across it (__syncthreads would also wait for every younger stage).
  // younger loads allowed in flight at a k-step's barrier / after the prologue (post-barrier
  // loads: none are issued between those the barrier waits for and the barrier; the prologue
  // issues both stages and waits for the first)
  constexpr int VMC_LOOP = POSTW ? (POST_BA > 0 ? N_DMA : 0) : (NST >= 3 ? N_DMA * (NST - 3) + DPRE : 0);
  constexpr int VMC_PRO = POSTW ? N_DMA : N_DMA * (NST - 2);
  static_assert(NST >= 2, "the ring needs at least 2 stages");
  static_assert(VMC_LOOP <= 63 && VMC_PRO <= 63, "vmcnt range");
  auto ring_barrier = [&](auto vmc_c) __attribute__((always_inline)) {
    if constexpr (VST)  // the stage was written from registers: only LDS traffic to wait for
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(decltype(vmc_c)::value) : "memory");
  };
  // Loads for k-step kt + NST - 1 are issued during k-step kt.  Slice ks of a k-step consumes
  // fragment buffer (B0 + ks) & 1 and reads the next slice into the other one; with an odd
  // number of slices per k-step (one) the buffers alternate between k-steps, so k-steps come
  // in pairs of parity 0 and 1 (B0 = parity * KS).
  auto kstep = [&](int kt, auto par_c, auto full_c) __attribute__((always_inline)) {
    constexpr int B0 = (decltype(par_c)::value * KS) & 1;
    const char* cur = smem + (kt % NST) * TR::STAGE;
    const char* nxt = smem + ((kt + 1) % NST) * TR::STAGE;
    // the stage written by this k-step's loads and the k-step they load: NST - 1 ahead into the
    // stage k-step kt - 1 used (register staging: one more, the registers holding k-step kt + 1
    // on their way to dst; post-barrier loads: two ahead, into this k-step's own stage)
    char* dst = smem + ((POSTW ? kt : kt + NST - 1) % NST) * TR::STAGE;
    const int kl = (VST || POSTW) ? kt + 2 : kt + NST - 1;
    const KnSrc kr = kn_rsrc(kl);
    if constexpr (PAIR) pair_dst = smem + ((kt + (decltype(par_c)::value == 1 ? 4 : 2)) % NST) * TR::STAGE;
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      u32x4* A = fa[(B0 + ks) & 1];
      u32x4* B = fb[(B0 + ks) & 1];
      u32x4* RA = fa[(B0 + ks + 1) & 1];
      u32x4* RB = fb[(B0 + ks + 1) & 1];
      lgkm_fence(A, B);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (POSTW && POST_BA > 0) {
        // (KS == 2: ks is 0) the second slice's fragments are read first; then the first barrier
        // frees the stage
        using BA_ = std::integral_constant<int, POST_BA>;
        slice(T_{}, std::integral_constant<int, 0>{}, A, B, Z_{}, BA_{}, kl, dst, kr, cur, ks + 1, RA, RB, par_c, full_c);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        slice(F_{}, std::integral_constant<int, 0>{}, A, B, BA_{}, W_{}, kl, dst, kr, cur, ks + 1, RA, RB, par_c, full_c);
      } else if (ks == 0)
        slice(T_{}, std::integral_constant<int, 0>{}, A, B, Z_{}, W_{}, kl, dst, kr, cur, ks + 1, RA, RB, par_c, full_c);
      else if (ks == 1)
        slice(T_{}, std::integral_constant<int, NMMA>{}, A, B, Z_{}, W_{}, kl, dst, kr, cur, ks + 1, RA, RB, par_c, full_c);
      else
        slice(T_{}, std::integral_constant<int, 2 * NMMA>{}, A, B, Z_{}, W_{}, kl, dst, kr, cur, ks + 1, RA, RB, par_c, full_c);
    }
    constexpr int L = (B0 + KS - 1) & 1;  // buffer of the last slice
    constexpr int NX = (B0 + KS) & 1;     // buffer of the next k-step's first slice
    using GL = std::integral_constant<int, (KS - 1) * NMMA>;
    lgkm_fence(fa[L], fb[L]);
    __builtin_amdgcn_sched_barrier(0);
    slice(F_{}, GL{}, fa[L], fb[L], Z_{}, H_{}, kl, dst, kr, cur, 0, fa[NX], fb[NX], par_c, full_c);
    // with k-step pairs the stage needed next is the second of the pair begun three k-steps
    // before (even kt) or the first of the pair begun two k-steps before (odd kt); the counts
    // of younger loads are pair_sched's
    ring_barrier(std::integral_constant<int, !PAIR ? VMC_LOOP : (decltype(par_c)::value == 0 ? PS_.vmc_even : PS_.vmc_odd)>{});
    __builtin_amdgcn_sched_barrier(0);
    slice(T_{}, GL{}, fa[L], fb[L], H_{}, W_{}, kl, dst, kr, nxt, 0, fa[NX], fb[NX], par_c, full_c);
  };
  using P0_ = std::integral_constant<int, 0>;
  using P1_ = std::integral_constant<int, 1>;

  if constexpr (MODE != 2) {
    if constexpr (VST) {
      // k-step 0 through the registers into stage 0, then k-step 1 into the registers
      const KnSrc k0 = kn_rsrc(0);
#pragma unroll
      for (int t = 0; t < N_DMA; ++t) sreg[t] = gload(0, t, k0);
#pragma unroll
      for (int t = 0; t < N_DMA; ++t) lput(smem, t);
      const KnSrc k1 = kn_rsrc(1);
#pragma unroll
      for (int t = 0; t < N_DMA; ++t) sreg[t] = gload(1, t, k1);
    } else {
      if constexpr (PAIR) {
        // k-steps 0 and 1, k-step 2's unpaired slots, then the first pafter loads of the
        // pair (2, 3), which k-step 0 completes as if the pair had been begun in k-step -1
        issue_tile(0, smem);
        issue_tile(1, smem + TR::STAGE);
        const KnSrc k2 = kn_rsrc(2);
#pragma unroll
        for (int j = 0; j < NU; ++j) dma_op(2, smem + 2 * TR::STAGE, NPS + j, k2, std::false_type{});
#pragma unroll
        for (int d = 0; d < PS_.pafter; ++d) dma_op(2 + (d & 1), smem + (2 + (d & 1)) * TR::STAGE, d >> 1, k2, std::false_type{});
      } else {
#pragma unroll
        for (int s = 0; s < (POSTW ? NST : NST - 1); ++s) issue_tile(s, smem + s * TR::STAGE);
      }
    }
    ring_barrier(std::integral_constant<int, PAIR ? PS_.vmc_pro : VMC_PRO>{});
    // the same wait, visible to the compiler (the barrier's is inline asm): with no scalar
    // or LDS load of its own in flight at the K loop's entry, its waits inside the loop
    // count the fragment reads exactly instead of waiting for all of them
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt not waited for
    __builtin_amdgcn_sched_barrier(0);
    read_frags(smem, 0, fa[0], fb[0]);
    if constexpr (KS % 2 == 0) {
      for (int kt = 0; kt < KT; ++kt) kstep(kt, P0_{}, F_{});
    } else {
      // k-steps in pairs; an odd count gets one more k-step, whose loads lie past the block's
      // K range and read as zeros, so that the loop has a single body (a separate last k-step
      // makes the register allocator move the accumulators between register files)
      for (int kt = 0; kt < KT; kt += 2) {
        kstep(kt, P0_{}, F_{});
        kstep(kt + 1, P1_{}, F_{});
      }
    }
  }
  // loads issued past the last k-step (they read as zeros) must land before LDS is reused
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (MF == 16) mfma_drain();
  lgkm_fence(fa[0], fb[0]);
  lgkm_fence(fa[1], fb[1]);
  __syncthreads();

  // ---------------------------------------------------------------- split-K
  // Partials are stored register-major: f32x4 number q of thread t of a tile's partial sits at
  // float offset (q * 256 + t) * 4, so each store / load instruction covers 1 KiB contiguously.
  constexpr int ACC4 = MB * NB * (ACC_R / 4);  // f32x4 accumulator groups per thread
  if constexpr (MODE == 1) {
    float* dst = p.part + ((int64_t)split * nsplit + (tbid - p.tail0)) * (int64_t)(ACC4 * kThreads * 4);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int g = 0; g < ACC_R / 4; ++g) {
          const int q = (i * NB + j) * (ACC_R / 4) + g;
          f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          __builtin_nontemporal_store(v, (f32x4*)(dst + ((int64_t)q * kThreads + tid) * 4));
        }
    return;
  } else {
  if constexpr (MODE == 2) {
    // the partials are summed in split order (so the result does not depend on which split
    // finished first), QB f32x4 groups at a time: the group's loads of one split are all
    // issued before they are added, so that a batch costs one memory latency per split
    // rather than one per load, and only the accumulators already summed are live
    constexpr int QB = cfg_occ(CFG) > 1 ? (ACC4 < 8 ? ACC4 : 8) : (ACC4 < 16 ? ACC4 : 16);  // (2 workgroups per CU: half the registers)
    static_assert(ACC4 % QB == 0, "accumulator groups per batch");
    constexpr int GPB = ACC_R / 4;  // f32x4 groups per MFMA block
    const float* src = p.part + (int64_t)(tbid - p.tail0) * (ACC4 * kThreads * 4) + tid * 4;
    const int64_t sstride = (int64_t)nsplit * (ACC4 * kThreads * 4);
#pragma unroll
    for (int q0 = 0; q0 < ACC4; q0 += QB) {
      f32x4 sum[QB];
#pragma unroll
      for (int u = 0; u < QB; ++u) sum[u] = __builtin_nontemporal_load((const f32x4*)(src + (int64_t)(q0 + u) * kThreads * 4));
      for (int sp = 1; sp < p.splits; ++sp) {
        f32x4 t[QB];
#pragma unroll
        for (int u = 0; u < QB; ++u)
          t[u] = __builtin_nontemporal_load((const f32x4*)(src + sp * sstride + (int64_t)(q0 + u) * kThreads * 4));
#pragma unroll
        for (int u = 0; u < QB; ++u) sum[u] += t[u];
      }
#pragma unroll
      for (int u = 0; u < QB; ++u) {
        const int q = q0 + u;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[q / GPB / NB][q / GPB % NB][4 * (q % GPB) + e] = sum[u][e];
      }
    }
  }

  // ---------------------------------------------------------------- epilogue
  // Accumulator layout: lane l of 32x32 block (i, j) holds column 32 j + l%32 of the wave's
  // columns and, in register r, row 8 (r/4) + 4 (l/32) + r%4 of the block's 32 rows; lane l
  // of 16x16 block (i, j) holds column 16 j + l%16 and, in register r, row 4 (l/16) + r.
  // Everything that needs only the column (bias, ReLU, the mask bits, SiLU*mul, the masked
  // column sums) is applied to the accumulators in place; then each 32-row slab is staged
  // through LDS so that every lane owns 8 consecutive columns of one row for the stores.
  constexpr int NBO = TR::NBO;
  constexpr bool HAS_BIAS = EPI == E_BIAS || EPI == E_RELU_BIAS || EPI == E_RELU_AUX_BIAS ||
                           EPI == E_GELU_BIAS || EPI == E_GELU_AUX_BIAS;
  constexpr bool BGRAD = EPI == E_DRELU_BGRAD || EPI == E_DGELU_BGRAD;
  constexpr bool RELU = EPI == E_RELU_BIAS || EPI == E_RELU_AUX_BIAS;
  const int l32 = lane & 31;
  const int lmf = lane & (MF - 1);
  const int q4 = lane >> 4;
  const int ccol0 = n0 + wn * WTN;  // first output column of the wave
  float* stg = (float*)smem + wave * TR::STG_FLOATS;
  constexpr int SP = TR::SPITCH;
  const int lr = lane / TR::LPR;        // staged row within an iteration
  const int lc = (lane % TR::LPR) * 8;  // first of the lane's 8 staged columns
  const int gcol = ccol0 + lc;
  const bool colok = gcol < N;

  float bias_mf[NBO];
#pragma unroll
  for (int j = 0; j < NBO; ++j) {
    bias_mf[j] = 0.0f;
    if constexpr (HAS_BIAS) {
      const int c = ccol0 + MF * j + lmf;
      if (c < N) bias_mf[j] = E::to_f32(((const uint16_t*)p.bias)[c]);
    }
  }
  f32x4 colsum[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};  // bias gradients: the lane's 8 columns

  // DSWIGLU reads gate and up, and DGELU_BGRAD the pre-activation, per element in the staged
  // layout one slab ahead (two buffers): slab 0 right after the K loop, slab i + 1 while slab
  // i is staged and stored, so that their latency passes behind the work of a whole slab.
  // (DSWIGLU with two workgroups per CU has the registers for one buffer only: it reads a
  // slab's gate and up when the slab begins, so that they arrive during its staging.)
  constexpr int PF_GU = (EPI == E_DSWIGLU || EPI == E_DGELU_BGRAD) ? TR::ITERS : 1;
  constexpr int GUB = (EPI == E_DSWIGLU && cfg_occ(CFG) == 1) ? 2 : 1;  // gate / up buffers
  u32x4 pf_g[GUB][PF_GU], pf_u[GUB][PF_GU];
  u32x4 pf_a[EPI == E_DGELU_BGRAD ? 2 : 1][PF_GU];
  // The epilog's row-wise inputs and outputs (the output d; DSWIGLU's gate, up and d_up; the
  // GELU pre-activation) go through buffer descriptors, one per 32-row slab, whose extent
  // ends with the slab's last row inside M: rows past M then read as zeros and their stores
  // are dropped by the hardware's range check (which covers the per-lane offset),
  // and lanes whose 8 columns lie past N (N is a multiple of 8) use an offset beyond every
  // extent.  The descriptors are wave-uniform (scalar), so a row costs one offset addition.
  // (Leading dimensions are below 2^22 elements, so every offset fits in 32 bits; with no row
  // inside M the extent (rc - 1) * ld2 + 2 N is at most 0, as ld >= N.)
  auto slab_rsrc = [&](const void* base, int64_t ld, int i) __attribute__((always_inline)) {
    const int srow0 = __builtin_amdgcn_readfirstlane(m0 + wm * WTM + i * 32);
    const int ld2 = (int)ld * 2;
    const int rc = min(max(M - srow0, 0), 32);  // rows of the slab inside M
    const uint32_t num = (uint32_t)max((rc - 1) * ld2 + N * 2, 0);
    // the base and extent read from lane 0: the compiler then keeps the descriptor in scalar
    // registers (it otherwise wraps some buffer instructions in a per-lane loop)
    const uint64_t a = (uint64_t)((const char*)base + (int64_t)srow0 * ld2);
    const uint64_t au = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    return make_rsrc_raw((const void*)au, (uint32_t)__builtin_amdgcn_readfirstlane((int)num));
  };
  constexpr uint32_t kOffNone = 0x80000000u;  // beyond every extent above (each is under 2^29)
  const uint32_t vo_gu = colok ? (uint32_t)(lr * p.ld_gu + gcol) * 2u : kOffNone;
  const uint32_t vo_d = colok ? (uint32_t)(lr * p.ldd + gcol) * 2u : kOffNone;
  const uint32_t vo_d2 = colok ? (uint32_t)(lr * p.ldd2 + gcol) * 2u : kOffNone;
  const uint32_t vo_ga = colok ? (uint32_t)(lr * p.ld_gaux + gcol) * 2u : kOffNone;
  auto load_gaux = [&](int i, u32x4* dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ra = slab_rsrc(p.gaux, p.ld_gaux, i);
#pragma unroll
    for (int it = 0; it < TR::ITERS; ++it)
      dst[it] = __builtin_amdgcn_raw_buffer_load_b128(ra, vo_ga + (uint32_t)(it * TR::RPI * (int)p.ld_gaux * 2), 0, 2);
  };
  auto load_gu = [&](int i, u32x4* g, u32x4* u) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rg = slab_rsrc(p.gate, p.ld_gu, i), ru = slab_rsrc(p.up, p.ld_gu, i);
#pragma unroll
    for (int it = 0; it < TR::ITERS; ++it) {
      const uint32_t vo = vo_gu + (uint32_t)(it * TR::RPI * (int)p.ld_gu * 2);
      // cache policy 2: non-temporal (each element is read once)
      g[it] = __builtin_amdgcn_raw_buffer_load_b128(rg, vo, 0, 2);
      u[it] = __builtin_amdgcn_raw_buffer_load_b128(ru, vo, 0, 2);
    }
  };
  if constexpr (EPI == E_DGELU_BGRAD) load_gaux(0, pf_a[0]);
  if constexpr (EPI == E_DSWIGLU && GUB == 2) load_gu(0, pf_g[0], pf_u[0]);

  // 32-row slabs: 32x32 block row i, or 16x16 block rows 2i and 2i + 1
#pragma unroll
  for (int i = 0; i < WTM / 32; ++i) {
    const int srow0 = m0 + wm * WTM + i * 32;  // first row of the slab
    uint32_t pf_w[NW];
    if constexpr (EPI == E_DRELU_BGRAD) {
#pragma unroll
      for (int q = 0; q < NW; ++q) pf_w[q] = mw_all[i][q];
    } else if constexpr (EPI == E_DGELU_BGRAD) {
      if (i + 1 < NSLAB) load_gaux(i + 1, pf_a[(i + 1) & 1]);
    } else if constexpr (EPI == E_DSWIGLU) {
      if constexpr (GUB == 2) {
        if (i + 1 < NSLAB) load_gu(i + 1, pf_g[(i + 1) & 1], pf_u[(i + 1) & 1]);
      } else {
        load_gu(i, pf_g[0], pf_u[0]);
      }
    }

    // ---- accumulator space, then the slab is staged
    uint32_t* mk = (uint32_t*)(smem + TR::MASK_OFF) + wm * 32 * TR::WPT;  // [32 rows][WPT words]
    constexpr bool XFORM = HAS_BIAS || DUAL;
    // one accumulator value of the epilog's column transform (bias, ReLU, SiLU * up)
    auto xform = [&](const AccT* arow, int j, int r, bool& pr) __attribute__((always_inline)) {
      float v;
      // (16x16 accumulators come from asm MFMAs: read one at a time, or the compiler copies
      // all of them out of the AGPRs at once)
      if constexpr (XFORM || MF == 16) v = acc_read(arow[j][r]);
      else v = arow[j][r];
      if constexpr (HAS_BIAS) v += bias_mf[j];
      pr = v > 0.0f;
      if constexpr (RELU) {
        v = pr ? v : 0.0f;
      } else if constexpr (DUAL) {
        // block j holds the gate columns, block j + NB/2 the up columns of the same outputs
        const float u = acc_read(arow[j + NB / 2][r]);
        v = v * sigmoid_f(v) * u;
      }
      return v;
    };
    if constexpr (MF == 32) {
#pragma unroll
      for (int j = 0; j < NBO; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int r0 = 8 * (r >> 2) + (r & 3);  // block row held by lanes 0-31 (lanes 32-63: +4)
          bool pr;
          const float v = xform(acc[i], j, r, pr);
          // staged right away (row 8 (r/4) + 4 (l/32) + r%4 of the slab, column 32 j + l%32)
          stg[(r0 + 4 * hlf) * SP + j * 32 + l32] = v;
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int jw = 0; jw < NBO / 2; ++jw)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            bool pr0, pr1;
            const float v0 = xform(acc[2 * i + h], 2 * jw, r, pr0);
            const float v1 = xform(acc[2 * i + h], 2 * jw + 1, r, pr1);
            const int srow = 16 * h + 4 * q4 + r;
            stg[srow * SP + 2 * jw * 16 + lmf] = v0;
            stg[srow * SP + (2 * jw + 1) * 16 + lmf] = v1;
          }
    }

    __syncthreads();

    // RELU_AUX_BIAS: the slab's mask words, gathered in LDS by the store loop below, go to
    // relu_aux after it (store_mask)
    auto store_mask = [&]() __attribute__((always_inline)) {
      // the tile's words of the slab's 32 rows: one contiguous piece of WPT words per row,
      // written by the wn = 0 wave (words past ceil(N / 32) are not part of the row)
      if (wn == 0) {
        constexpr int LPRW = TR::WPT / 4;  // lanes per row, 4 words (16 bytes) each
        const int nw = (N + 31) / 32;
        const bool vec = (((uintptr_t)p.aux_out | (uintptr_t)(p.ld_aux * 4)) & 15) == 0;
#pragma unroll
        for (int pass = 0; pass < (32 * LPRW + 63) / 64; ++pass) {
          const int t = pass * 64 + lane;
          const int row = t / LPRW, part = t % LPRW;
          const int grow = srow0 + row;
          const int w0 = n0 / 32 + part * 4;
          if (row < 32 && grow < M && w0 < nw) {
            const u32x4 v = *(const u32x4*)(mk + row * TR::WPT + part * 4);
            uint32_t* dst = p.aux_out + (int64_t)grow * p.ld_aux + w0;
            if (vec && w0 + 4 <= nw) {
              *(u32x4*)dst = v;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (w0 + e < nw) dst[e] = v[e];
            }
          }
        }
      }
    };

    // ---- stores: CH staged rows per chunk, their LDS reads issued together
    // (the lane's output address of staged row 0; staged row t is t * ldd elements further)
    char* const dslab = (char*)p.d + ((int64_t)(srow0 + lr) * p.ldd + gcol) * 2;
    // DSWIGLU: the slab's d_gate and d_up rows (unused by the other epilogs)
    const __amdgpu_buffer_rsrc_t rs_d = slab_rsrc(p.d, p.ldd, i), rs_d2 = slab_rsrc(p.d2, p.ldd2, i);
    constexpr int OUTER_UNROLL = EPI == E_DRELU_BGRAD ? 2 : TR::ITERS;
#pragma unroll OUTER_UNROLL
    for (int c0 = 0; c0 < TR::ITERS; c0 += TR::CH) {
      f32x4 vv[TR::CH][2];
#pragma unroll
      for (int c = 0; c < TR::CH; ++c) {
        const float* src = stg + ((c0 + c) * TR::RPI + lr) * SP + lc;
        vv[c][0] = *(const f32x4*)src;
        vv[c][1] = *(const f32x4*)(src + 4);
      }
      if constexpr (EPI == E_DRELU_BGRAD) {
        uint32_t wd[TR::CH];
#pragma unroll
        for (int c = 0; c < TR::CH; ++c) {
          const int lrow = (c0 + c) * TR::RPI + lr;
          const int q = ((c0 + c) * TR::RPI) / RPW;  // the same for every lane of the row group
          const uint32_t src = NW == 1 ? pf_w[0] : (q ? pf_w[NW - 1] : pf_w[0]);
          wd[c] = (uint32_t)__shfl((int)src, (lrow % RPW) * WPR + (lc >> 5)) >> (gcol & 31);
        }
#pragma unroll
        for (int c = 0; c < TR::CH; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            // bit e of the word, sign-extended to all ones or zero, keeps the value or makes it
            // +0 (the element is copied out first: a bit cast of a vector-element lvalue reads
            // the vector's first element)
            const uint32_t keep = (uint32_t)((int32_t)(wd[c] << (31 - e)) >> 31);
            vv[c][e >> 2][e & 3] = __uint_as_float(and_opaque(__float_as_uint(vv[c][e >> 2][e & 3]), keep));
          }
      }
#pragma unroll
      for (int c = 0; c < TR::CH; ++c) {
        const int grow = srow0 + (c0 + c) * TR::RPI + lr;
        const bool ok = colok && grow < M;
        char* const dptr = dslab + (int64_t)((c0 + c) * TR::RPI) * p.ldd * 2;
        if constexpr (EPI == E_DSWIGLU) {
          {
            f32x4 dg[2], du[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const f32x4 g = unpack4<DT>(u32x2{pf_g[i % GUB][c0 + c][2 * h], pf_g[i % GUB][c0 + c][2 * h + 1]});
              const f32x4 u = unpack4<DT>(u32x2{pf_u[i % GUB][c0 + c][2 * h], pf_u[i % GUB][c0 + c][2 * h + 1]});
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float sg = sigmoid_f(g[e]);
                const float t = vv[c][h][e] * sg;        // dh * s
                du[h][e] = t * g[e];                     // dh * silu(g)
                dg[h][e] = t * u[e] * (1.0f + g[e] * (1.0f - sg));
              }
            }
            // (rows past M and columns past N are dropped by the range check.)  Cache policy 2,
            // non-temporal: d_gate and d_up stream out instead of displacing from L2 the operand
            // lines that the running tiles' K loops share (16384 x 17408 x 5120 on MI355X: about
            // 2 % faster than write-back stores; other epilogs measured no consistent gain)
            const int rr = (c0 + c) * TR::RPI;
            __builtin_amdgcn_raw_buffer_store_b128(pack8<DT>(dg[0], dg[1]), rs_d, vo_d + (uint32_t)(rr * (int)p.ldd * 2), 0, 2);
            __builtin_amdgcn_raw_buffer_store_b128(pack8<DT>(du[0], du[1]), rs_d2, vo_d2 + (uint32_t)(rr * (int)p.ldd2 * 2), 0, 2);
          }
        } else if constexpr (EPI == E_GELU_BIAS || EPI == E_GELU_AUX_BIAS) {
          {
            const int rr = (c0 + c) * TR::RPI;
            if constexpr (EPI == E_GELU_AUX_BIAS)
              __builtin_amdgcn_raw_buffer_store_b128(pack8<DT>(vv[c][0], vv[c][1]), slab_rsrc(p.gaux, p.ld_gaux, i),
                                                     vo_ga + (uint32_t)(rr * (int)p.ld_gaux * 2), 0, 0);
            f32x4 y[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int e = 0; e < 4; ++e) y[h][e] = gelu_f(vv[c][h][e]);
            __builtin_amdgcn_raw_buffer_store_b128(pack8<DT>(y[0], y[1]), rs_d, vo_d + (uint32_t)(rr * (int)p.ldd * 2), 0, 0);
          }
        } else {
          if constexpr (EPI == E_DGELU_BGRAD) {  // rows past M: aux read as 0, staged value 0
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const f32x4 pa = unpack4<DT>(u32x2{pf_a[i & 1][c0 + c][2 * h], pf_a[i & 1][c0 + c][2 * h + 1]});
#pragma unroll
              for (int e = 0; e < 4; ++e) vv[c][h][e] *= gelu_grad_f(pa[e]);
            }
          }
          __builtin_amdgcn_raw_buffer_store_b128(pack8<DT>(vv[c][0], vv[c][1]), rs_d,
                                                 vo_d + (uint32_t)((c0 + c) * TR::RPI * (int)p.ldd * 2), 0, 0);
          if constexpr (EPI == E_RELU_AUX_BIAS) {
            // the mask bits of the lane's 8 columns: the staged values are ReLU's output, which
            // is +0 exactly where the pre-activation is not > 0 (NaN included) and positive
            // elsewhere, so bit e is (bits of value e != 0).  They make byte (lane % LPR) of the
            // wave's piece of the row (LSB = lowest column; columns past N were staged as +0).
            uint32_t byte = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) byte |= min(__float_as_uint(vv[c][e >> 2][e & 3]), 1u) << e;
            ((unsigned char*)(mk + ((c0 + c) * TR::RPI + lr) * TR::WPT + wn * WPR))[lane % TR::LPR] = (unsigned char)byte;
          }
          if constexpr (BGRAD) {  // rows past M are staged as 0
            colsum[0] += vv[c][0];
            colsum[1] += vv[c][1];
            // the running sums are taken here: left free, the compiler sank every addition to
            // the end of the epilogue and kept each row's values live until then (spills)
            asm volatile("" : "+v"(colsum[0]), "+v"(colsum[1]));
          }
        }
      }
    }
    __syncthreads();
    if constexpr (EPI == E_RELU_AUX_BIAS) store_mask();

    if constexpr (EPI == E_SWIGLU_AUX) {
      // the gate (pass 0) and up (pass 1) pre-activations of the slab, still in the
      // accumulators, go to d2 columns [0, N) and [N, 2N)
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        if constexpr (MF == 32) {
#pragma unroll
          for (int j = 0; j < NBO; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int r0 = 8 * (r >> 2) + (r & 3);
              stg[(r0 + 4 * hlf) * SP + j * 32 + l32] = pass == 0 ? acc[i][j][r] : acc[i][j + NB / 2][r];
            }
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < NBO; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                stg[(16 * h + 4 * q4 + r) * SP + j * 16 + lmf] =
                    acc_read(pass == 0 ? acc[2 * i + h][j][r] : acc[2 * i + h][j + NB / 2][r]);
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < TR::ITERS; ++it) {
          const int grow = srow0 + it * TR::RPI + lr;
          const float* src = stg + (it * TR::RPI + lr) * SP + lc;
          const f32x4 v0 = *(const f32x4*)src, v1 = *(const f32x4*)(src + 4);
          if (colok && grow < M)
            *(u32x4*)((char*)p.d2 + ((int64_t)grow * p.ldd2 + pass * N + gcol) * 2) = pack8<DT>(v0, v1);
        }
        __syncthreads();
      }
    }
  }

  if constexpr (BGRAD) {
    // lanes that share columns: lane, lane + LPR, ... (different rows); then the other
    // M-wave's sums through LDS; one partial per (M tile, column), or an atomic add
#pragma unroll
    for (int sh = TR::LPR; sh < 64; sh <<= 1)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) colsum[h][e] += __shfl_xor(colsum[h][e], sh);
    float* bg = (float*)(smem + TR::BG_OFF) + wn * WTN;
    if (wm == 1 && lane < TR::LPR) {
      *(f32x4*)(bg + lc) = colsum[0];
      *(f32x4*)(bg + lc + 4) = colsum[1];
    }
    __syncthreads();
    if (wm == 0 && lane < TR::LPR && colok) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 tot = colsum[h] + *(const f32x4*)(bg + lc + 4 * h);
        if (p.bgrad_atomic) {
#pragma unroll
          for (int e = 0; e < 4; ++e) atomicAdd(p.bgrad_part + gcol + 4 * h + e, tot[e]);
        } else {
          *(f32x4*)(p.bgrad_part + (int64_t)pm * N + gcol + 4 * h) = tot;
        }
      }
    }
  }
}  // MODE != 1
}

template <int DT, int LAY, int EPI, int CFG, int MODE = 0>
void launch_gemm(const GemmArgs& a, hipStream_t s) {
  const int ntiles = a.tiles_m * a.tiles_n;
  // MODE 0 runs every tile, or the whole-K tiles [0, tail0) of a split plan
  const int nblocks = MODE == 0 ? (a.splits > 1 ? a.tail0 : ntiles) : (ntiles - a.tail0) * (MODE == 1 ? a.splits : 1);
  hipLaunchKernelGGL((gemm_kernel<DT, LAY, EPI, CFG, MODE>), dim3(nblocks), dim3(kThreads), 0, s, a);
}

}  // namespace ep
