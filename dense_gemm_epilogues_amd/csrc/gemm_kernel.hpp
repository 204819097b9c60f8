// Fused GEMM + epilogue kernel for CDNA4 (gfx950).
//
// One workgroup (4 wave64s in a 2x2 grid) computes a BM x BN output tile:
//   * A and B tiles of 64 k-values are staged in LDS, double buffered, in a k-contiguous
//     layout (each row = 64 elements = 128 bytes = 8 chunks of 16 bytes) with chunk c of row
//     r stored at chunk c ^ ((r ^ r>>3) & 7), so that every 8 (and 16) consecutive rows read
//     by the MFMA fragment loads hit distinct banks.
//   * Global loads are 16-byte buffer loads (hardware bounds checks give zeros past the
//     matrix edges).  A B operand given K x N (N contiguous) is transposed in registers
//     (8 k-rows x 8 columns per thread) before it is written to LDS, so both B layouts
//     share one LDS layout and one fragment-read path.
//   * The K loop issues v_mfma_f32_32x32x16_{f16,bf16}: lane l of a 32x32 block holds
//     column l%32 and rows 8*(r/4) + 4*(l/32) + r%4 of its 16 accumulator registers.
//   * The epilogue runs on the float32 accumulators: each wave stages a 32-row slab through
//     LDS so that every lane owns 4 consecutive columns of one row, applies the epilog
//     (bias, ReLU, mask packing, mask application + column sums, SiLU*mul, dSwiGLU) in
//     float32 and writes each output once, with 8-byte row-contiguous stores.
//
// Epilogs follow "Fusing Matmul Epilogs with nvmath-python" (forward: RELU_BIAS,
// RELU_AUX_BIAS; backward: DRELU_BGRAD), the hotdry.top cuBLASLt post (BIAS, the
// plan/execute split) and gemm_swiglu_mlp_fusion.py (SwiGLU forward, dSwiGLU epilogue).
#pragma once
#include "ep_internal.hpp"

namespace ep {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past every num_records we build

constexpr int cfg_bm(int cfg) { return cfg == 0 ? 256 : cfg == 1 ? 128 : cfg == 2 ? 256 : 128; }
constexpr int cfg_bnt(int cfg) { return cfg == 0 ? 256 : cfg == 1 ? 128 : cfg == 2 ? 128 : 256; }

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
};

template <int DT>
__device__ __forceinline__ u32x2 pack4(f32x4 v) {
  using E = Elem<DT>;
  u32x2 r;
  r[0] = E::from_f32(v[0]) | (E::from_f32(v[1]) << 16);
  r[1] = E::from_f32(v[2]) | (E::from_f32(v[3]) << 16);
  return r;
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

// Logistic function from its definition, 1 / (1 + e^-t), with e^-t = 2^(-t log2 e) on the
// hardware exp2.  t -> -inf gives 2^(+inf) = inf and 1/inf = 0; t -> +inf gives 1.
__device__ __forceinline__ float sigmoid_f(float t) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * t));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7fffffffLL ? 0x7fffffffu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// byte offset of 16-byte chunk `c` of row `r` in a k-contiguous LDS tile
__device__ __forceinline__ uint32_t swz(int r, int c) {
  return (uint32_t)(r * 128 + (((c ^ r ^ (r >> 3)) & 7) << 4));
}

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a contiguous range
// of the tile order so that tiles sharing A rows / B columns share that XCD's L2, and
// walk tiles in groups of kGroupM tile-rows.
__device__ __forceinline__ void map_tile(int bid, int nblocks, int tiles_m, int tiles_n, int& pm,
                                         int& pn) {
  const int q = nblocks >> 3, r = nblocks & 7;
  const int x = bid & 7, l = bid >> 3;
  const int t = (x < r) ? x * (q + 1) + l : r * (q + 1) + (x - r) * q + l;
  const int group = kGroupM * tiles_n;
  const int g = t / group;
  const int first_m = g * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int w = t - g * group;
  pm = first_m + w % gm;
  pn = w / gm;
}

template <int DT, int LAY, int EPI, int BM, int BNT>
struct GemmTraits {
  static constexpr bool DUAL = EPI == E_SWIGLU;
  static constexpr int WTM = BM / 2;             // rows per wave
  static constexpr int WTB = BNT / 2;            // B-tile rows per wave
  static constexpr int MB = WTM / 32;            // 32x32 blocks per wave along M
  static constexpr int NB = WTB / 32;            // ... along the B tile
  static constexpr int BN_OUT = DUAL ? BNT / 2 : BNT;
  static constexpr int WTN = DUAL ? WTB / 2 : WTB;  // output columns per wave
  static constexpr int A_BYTES = BM * 128;
  static constexpr int B_BYTES = BNT * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_PER = BM / 32;          // 16-byte chunks per thread per k-step
  static constexpr int B_PER = BNT / 32;
  static constexpr int SPITCH = WTN + 8;         // staging pitch in floats
  static constexpr int NARR = DUAL ? 2 : 1;
  static constexpr int STG_FLOATS = NARR * 32 * SPITCH;  // per wave
  static constexpr int BG_OFF = 4 * STG_FLOATS * 4;      // bytes; cross-wave bgrad exchange
  static constexpr int EPI_BYTES = BG_OFF + 2 * WTN * 4;
  static constexpr int LDS_BYTES = (2 * STAGE > EPI_BYTES) ? 2 * STAGE : EPI_BYTES;
  static constexpr int LPR = WTN / 4;            // lanes per staged row
  static constexpr int RPI = 64 / LPR;           // staged rows per iteration
  static constexpr int ITERS = 32 / RPI;
  static_assert(LPR >= 8 && LPR <= 64, "a relu_aux word must span whole lanes");
};

template <int DT, int LAY, int EPI, int BM, int BNT>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmArgs p) {
  using E = Elem<DT>;
  using TR = GemmTraits<DT, LAY, EPI, BM, BNT>;
  constexpr bool DUAL = TR::DUAL;
  constexpr int MB = TR::MB, NB = TR::NB, WTM = TR::WTM, WTB = TR::WTB, WTN = TR::WTN;
  constexpr int A_PER = TR::A_PER, B_PER = TR::B_PER;

  __shared__ __attribute__((aligned(16))) char smem[TR::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int pm, pn;
  map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, pm, pn);
  const int m0 = pm * BM;
  const int n0 = pn * TR::BN_OUT;
  const int M = p.M, N = p.N, K = p.K;
  const int KT = (K + kBK - 1) / kBK;

  const char* Ag = (const char*)p.a;
  const char* Bg = (const char*)p.b;
  const char* B2g = DUAL ? (const char*)p.b2 : (const char*)p.b;

  // ---------------------------------------------------------------- loader setup
  // A: chunk i of this thread is row i*32 + tid/8, 16-byte column chunk tid%8.
  uint32_t a_off[A_PER], a_lds[A_PER];
  const int ld_c = tid & 7;
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int row = i * 32 + (tid >> 3);
    a_off[i] = (uint32_t)(row * p.lda * 2) + ld_c * 16;
    a_lds[i] = swz(row, ld_c);
  }
  // B, N x K layout: like A over the BNT rows of the B tile (DUAL: first half Wg, second Wu).
  // B, K x N layout: thread owns KR consecutive k-rows of one 8-column chunk.
  constexpr int NCH = BNT / 8;              // 8-column chunks across the B tile
  constexpr int KR = (LAY == L_KN) ? BNT / 32 : 1;
  uint32_t b_off[B_PER], b_lds[B_PER];
  bool b_second[B_PER];
  int kn_b = 0, kn_g = 0;
  bool kn_colok = true;
  if constexpr (LAY == L_NK) {
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int row = i * 32 + (tid >> 3);
      const int srow = DUAL ? (row % (BNT / 2)) : row;
      b_second[i] = DUAL && row >= BNT / 2;
      b_off[i] = (uint32_t)(srow * p.ldb * 2) + ld_c * 16;
      b_lds[i] = swz(row, ld_c);
    }
  } else {
    kn_b = tid % NCH;
    kn_g = tid / NCH;
    const int sb = DUAL ? (kn_b % (NCH / 2)) : kn_b;
    const bool second = DUAL && kn_b >= NCH / 2;
    kn_colok = (n0 + sb * 8) < N;
#pragma unroll
    for (int r = 0; r < B_PER; ++r) {  // B_PER == KR for this layout
      b_second[r] = second;
      b_off[r] = (uint32_t)((kn_g * KR + r) * p.ldb * 2) + sb * 16;
      b_lds[r] = 0;
    }
  }

  u32x4 ra[A_PER], rb[B_PER];

  auto load_tile = [&](int kt) {
    const int k0 = kt * kBK;
    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(Ag + ((int64_t)m0 * p.lda + k0) * 2, ((int64_t)(M - m0) * p.lda - k0) * 2);
    const bool kok = (k0 + ld_c * 8) < K;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) ra[i] = bload16(rA, kok ? a_off[i] : kOOB);
    if constexpr (LAY == L_NK) {
      const int64_t bbytes = ((int64_t)(N - n0) * p.ldb - k0) * 2;
      const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bg + ((int64_t)n0 * p.ldb + k0) * 2, bbytes);
      const __amdgpu_buffer_rsrc_t rB2 = make_rsrc(B2g + ((int64_t)n0 * p.ldb + k0) * 2, bbytes);
#pragma unroll
      for (int i = 0; i < B_PER; ++i)
        rb[i] = bload16(b_second[i] ? rB2 : rB, kok ? b_off[i] : kOOB);
    } else {
      const int64_t bbytes = ((int64_t)(K - k0) * p.ldb - n0) * 2;
      const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bg + ((int64_t)k0 * p.ldb + n0) * 2, bbytes);
      const __amdgpu_buffer_rsrc_t rB2 = make_rsrc(B2g + ((int64_t)k0 * p.ldb + n0) * 2, bbytes);
#pragma unroll
      for (int r = 0; r < B_PER; ++r)
        rb[r] = bload16(b_second[r] ? rB2 : rB, kn_colok ? b_off[r] : kOOB);
    }
  };

  auto store_tile = [&](int st) {
    char* As = smem + st * TR::STAGE;
    char* Bs = As + TR::A_BYTES;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) *(u32x4*)(As + a_lds[i]) = ra[i];
    if constexpr (LAY == L_NK) {
#pragma unroll
      for (int i = 0; i < B_PER; ++i) *(u32x4*)(Bs + b_lds[i]) = rb[i];
    } else {
      // transpose KR k-rows x 8 columns: column j gets the KR halves of its k-rows
      const int kbase = kn_g * KR;
      const int c = kbase >> 3;
      const int sub = (kbase & 7) * 2;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int nr = kn_b * 8 + j;
        char* dst = Bs + swz(nr, c) + sub;
        uint32_t w[KR / 2];
#pragma unroll
        for (int q = 0; q < KR / 2; ++q) {
          const uint32_t lo = rb[2 * q][j >> 1], hi = rb[2 * q + 1][j >> 1];
          w[q] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        if constexpr (KR == 8) {
          *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
        } else if constexpr (KR == 4) {
          *(u32x2*)dst = u32x2{w[0], w[1]};
        } else {
          *(uint32_t*)dst = w[0];
        }
      }
    }
  };

  // fragment-read rows
  const int hlf = lane >> 5;
  uint32_t a_rd[MB], b_rd[NB];
  int a_f[MB], b_f[NB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int row = wm * WTM + i * 32 + (lane & 31);
    a_rd[i] = row * 128;
    a_f[i] = (row ^ (row >> 3)) & 7;
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    int brow;
    if constexpr (DUAL) {
      brow = (j < NB / 2) ? wn * (WTB / 2) + j * 32 : BNT / 2 + wn * (WTB / 2) + (j - NB / 2) * 32;
    } else {
      brow = wn * WTB + j * 32;
    }
    const int row = brow + (lane & 31);
    b_rd[j] = row * 128;
    b_f[j] = (row ^ (row >> 3)) & 7;
  }

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---------------------------------------------------------------- main loop
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < KT) load_tile(kt + 1);
    const char* As = smem + st * TR::STAGE;
    const char* Bs = As + TR::A_BYTES;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      u32x4 af[MB], bf[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        af[i] = *(const u32x4*)(As + a_rd[i] + ((((ks * 2 + hlf) ^ a_f[i]) & 7) << 4));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        bf[j] = *(const u32x4*)(Bs + b_rd[j] + ((((ks * 2 + hlf) ^ b_f[j]) & 7) << 4));
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = E::mfma(af[i], bf[j], acc[i][j]);
    }
    if (kt + 1 < KT) store_tile(st ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  float* stg = (float*)smem + wave * TR::STG_FLOATS;
  constexpr int SP = TR::SPITCH;
  constexpr int NBO = DUAL ? NB / 2 : NB;  // blocks per staged array
  const int lr = lane / TR::LPR;           // row within an iteration
  const int lc = (lane % TR::LPR) * 4;     // staged column
  const int gcol = n0 + wn * WTN + lc;
  const bool colok = gcol < N;

  f32x4 bias4 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (EPI == E_BIAS || EPI == E_RELU_BIAS || EPI == E_RELU_AUX_BIAS) {
    if (colok) bias4 = unpack4<DT>(*(const u32x2*)((const char*)p.bias + (int64_t)gcol * 2));
  }
  f32x4 colsum = {0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      float* arr = stg + (DUAL ? (j / NBO) * 32 * SP : 0);
      const int col = (j % NBO) * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * hlf + (r & 3);
        arr[row * SP + col] = acc[i][j][r];
      }
    }
    __syncthreads();
#pragma unroll 2
    for (int it = 0; it < TR::ITERS; ++it) {
      const int lrow = it * TR::RPI + lr;
      const int grow = m0 + wm * WTM + i * 32 + lrow;
      const bool ok = colok && grow < M;
      f32x4 v = *(const f32x4*)(stg + lrow * SP + lc);
      const int64_t drow = (int64_t)grow * p.ldd;
      if constexpr (EPI == E_DEFAULT) {
        if (ok) *(u32x2*)((char*)p.d + (drow + gcol) * 2) = pack4<DT>(v);
      } else if constexpr (EPI == E_BIAS) {
        v += bias4;
        if (ok) *(u32x2*)((char*)p.d + (drow + gcol) * 2) = pack4<DT>(v);
      } else if constexpr (EPI == E_RELU_BIAS || EPI == E_RELU_AUX_BIAS) {
        v += bias4;
        uint32_t nib = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool pr = v[e] > 0.0f;
          v[e] = pr ? v[e] : 0.0f;
          nib |= (pr ? 1u : 0u) << e;
        }
        if (ok) *(u32x2*)((char*)p.d + (drow + gcol) * 2) = pack4<DT>(v);
        if constexpr (EPI == E_RELU_AUX_BIAS) {
          uint32_t w = (colok ? nib : 0u) << (4 * (lane & 7));
          w |= (uint32_t)__shfl_xor((int)w, 1);
          w |= (uint32_t)__shfl_xor((int)w, 2);
          w |= (uint32_t)__shfl_xor((int)w, 4);
          if (ok && (lane & 7) == 0) p.aux_out[(int64_t)grow * p.ld_aux + (gcol >> 5)] = w;
        }
      } else if constexpr (EPI == E_DRELU_BGRAD) {
        const uint32_t word = ok ? p.aux_in[(int64_t)grow * p.ld_aux + (gcol >> 5)] : 0u;
        const uint32_t bits = word >> (gcol & 31);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = ((bits >> e) & 1u) ? v[e] : 0.0f;
        if (ok) *(u32x2*)((char*)p.d + (drow + gcol) * 2) = pack4<DT>(v);
        colsum += v;
      } else if constexpr (EPI == E_SWIGLU) {
        const f32x4 u = *(const f32x4*)(stg + 32 * SP + lrow * SP + lc);
        f32x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = v[e] * sigmoid_f(v[e]) * u[e];
        if (ok) *(u32x2*)((char*)p.d + (drow + gcol) * 2) = pack4<DT>(h);
      } else if constexpr (EPI == E_DSWIGLU) {
        if (ok) {
          const int64_t go = ((int64_t)grow * p.ld_gu + gcol) * 2;
          const f32x4 g = unpack4<DT>(*(const u32x2*)((const char*)p.gate + go));
          const f32x4 u = unpack4<DT>(*(const u32x2*)((const char*)p.up + go));
          f32x4 dg, du;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float s = sigmoid_f(g[e]);
            const float t = v[e] * s;             // dh * s
            du[e] = t * g[e];                     // dh * silu(g)
            dg[e] = t * u[e] * (1.0f + g[e] * (1.0f - s));
          }
          *(u32x2*)((char*)p.d + (drow + gcol) * 2) = pack4<DT>(dg);
          *(u32x2*)((char*)p.d2 + ((int64_t)grow * p.ldd2 + gcol) * 2) = pack4<DT>(du);
        }
      }
    }
    __syncthreads();
  }

  if constexpr (EPI == E_DRELU_BGRAD) {
    // lanes that share columns: lane, lane + LPR, ... (different rows)
#pragma unroll
    for (int s = TR::LPR; s < 64; s <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) colsum[e] += __shfl_xor(colsum[e], s);
    float* bg = (float*)(smem + TR::BG_OFF) + wn * WTN;
    if (wm == 1 && lane < TR::LPR) *(f32x4*)(bg + lc) = colsum;
    __syncthreads();
    if (wm == 0 && lane < TR::LPR && colok) {
      const f32x4 other = *(const f32x4*)(bg + lc);
      const f32x4 tot = colsum + other;
      if (p.bgrad_atomic) {
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicAdd(p.bgrad_part + gcol + e, tot[e]);
      } else {
        *(f32x4*)(p.bgrad_part + (int64_t)pm * N + gcol) = tot;
      }
    }
  }
}

template <int DT, int LAY, int EPI, int CFG>
void launch_gemm(const GemmArgs& a, hipStream_t s) {
  constexpr int BM = cfg_bm(CFG), BNT = cfg_bnt(CFG);
  const int nblocks = a.tiles_m * a.tiles_n;
  hipLaunchKernelGGL((gemm_kernel<DT, LAY, EPI, BM, BNT>), dim3(nblocks), dim3(kThreads), 0, s, a);
}

#define EP_LAUNCH_ROW(DT, LAY, EPI) \
  { launch_gemm<DT, LAY, EPI, 0>, launch_gemm<DT, LAY, EPI, 1>, launch_gemm<DT, LAY, EPI, 2>, launch_gemm<DT, LAY, EPI, 3> }

#define EP_LAUNCH_TABLE(DT, LAY)                                                              \
  {                                                                                           \
    EP_LAUNCH_ROW(DT, LAY, E_DEFAULT), EP_LAUNCH_ROW(DT, LAY, E_BIAS),                        \
        EP_LAUNCH_ROW(DT, LAY, E_RELU_BIAS), EP_LAUNCH_ROW(DT, LAY, E_RELU_AUX_BIAS),         \
        EP_LAUNCH_ROW(DT, LAY, E_DRELU_BGRAD), EP_LAUNCH_ROW(DT, LAY, E_SWIGLU),              \
        EP_LAUNCH_ROW(DT, LAY, E_DSWIGLU)                                                     \
  }

}  // namespace ep
