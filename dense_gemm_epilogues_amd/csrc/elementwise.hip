// Unfused baseline kernels and the bias-gradient second pass.
//
// The unfused path reproduces the sequences the pages contrast with fusion: GEMM, then a
// separate bias addition and a separate ReLU ("The problem addressed by fused epilogs";
// the hotdry.top post's three-kernel comparison), GEMM then a manual mask and a batch sum
// ("Backward-pass path shown in the example"), two GEMMs then an activation kernel, and a
// GEMM followed by an elementwise dSwiGLU (gemm_swiglu_mlp_fusion.py docstring).  Each
// kernel is a plain HBM-bound pass: 16-byte row-contiguous accesses, one element group of
// 8 per thread, grid-stride loops.
#include "ep_internal.hpp"
#include "normal_dist.hpp"

namespace ep {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ float ld_f(uint32_t bits) {
  if constexpr (DT == T_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  else return __builtin_bit_cast(float, bits << 16);
}
template <int DT>
__device__ __forceinline__ uint32_t st_f(float x) {
  if constexpr (DT == T_F16) return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
  else return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}
template <int DT>
__device__ __forceinline__ void unpack8(u32x4 w, float* f) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = ld_f<DT>(w[q] & 0xffffu);
    f[2 * q + 1] = ld_f<DT>(w[q] >> 16);
  }
}
template <int DT>
__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 w;
#pragma unroll
  for (int q = 0; q < 4; ++q) w[q] = st_f<DT>(f[2 * q]) | (st_f<DT>(f[2 * q + 1]) << 16);
  return w;
}

__device__ __forceinline__ float sigmoid_f(float t) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * t));
}

// Row-tiled launch shape shared by the elementwise kernels: blockIdx.y walks rows (grid-stride
// past 65535; the row index is 64-bit, since a row count up to 2^31 - 1 plus the stride would
// overflow an int), blockIdx.x covers a row's 8-column groups, kGroups groups per thread,
// kEwThreads apart (each thread loads all of its groups before using any).  No integer division.
constexpr int kEwThreads = 256;
constexpr int kGroups = 2;

__device__ __forceinline__ int group_of(int u) {
  return (blockIdx.x * kGroups + u) * kEwThreads + threadIdx.x;
}

template <int DT>
__global__ void bias_add_kernel(char* z, int64_t ldz, const char* bias, int M, int N) {
  const int gpr = N / 8;
  for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
    char* zr = z + (int64_t)row * ldz * 2;
    u32x4 w[kGroups], bw[kGroups];
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
      const int g = group_of(u);
      if (g < gpr) {
        w[u] = *(const u32x4*)(zr + g * 16);
        bw[u] = *(const u32x4*)(bias + g * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
      const int g = group_of(u);
      if (g < gpr) {
        float f[8], b[8];
        unpack8<DT>(w[u], f);
        unpack8<DT>(bw[u], b);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] += b[e];
        *(u32x4*)(zr + g * 16) = pack8<DT>(f);
      }
    }
  }
}

// Y = relu(Z); with_mask: also the relu_aux words.  One thread per 8 columns; the 4 threads
// of a 32-column word are consecutive lanes (kEwThreads is a multiple of 4) and combine their
// bytes with lane shuffles.  Groups run to a whole number of words per row (gpr = 4 nw).
template <int DT>
__global__ void relu_pack_kernel(const char* z, int64_t ldz, char* y, int64_t ldy, uint32_t* aux,
                                 int64_t ld_aux, int M, int N, int with_mask) {
  const int nw = (N + 31) / 32;
  const int gpr = nw * 4;
  for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
    const char* zr = z + (int64_t)row * ldz * 2;
    char* yr = y + (int64_t)row * ldy * 2;
    u32x4 w[kGroups];
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
      const int g = group_of(u);
      if (g < gpr && g * 8 < N) w[u] = *(const u32x4*)(zr + g * 16);
    }
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
      const int g = group_of(u);
      uint32_t byte = 0;
      if (g < gpr && g * 8 < N) {
        float f[8];
        unpack8<DT>(w[u], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool pr = f[e] > 0.0f;
          byte |= (pr ? 1u : 0u) << e;
          f[e] = pr ? f[e] : 0.0f;
        }
        *(u32x4*)(yr + g * 16) = pack8<DT>(f);
      }
      if (with_mask) {  // every lane takes part in the shuffles
        uint32_t mw = byte << (8 * (threadIdx.x & 3));
        mw |= (uint32_t)__shfl_xor((int)mw, 1);
        mw |= (uint32_t)__shfl_xor((int)mw, 2);
        if (g < gpr && (threadIdx.x & 3) == 0) aux[(int64_t)row * ld_aux + (g >> 2)] = mw;
      }
    }
  }
}

template <int DT>
__global__ void mask_apply_kernel(const char* gsrc, int64_t ldg, const uint32_t* aux, int64_t ld_aux,
                                  char* dx, int64_t lddx, int M, int N) {
  const int gpr = N / 8;
  for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
    const char* gr = gsrc + (int64_t)row * ldg * 2;
    const uint32_t* ar = aux + (int64_t)row * ld_aux;
    u32x4 w[kGroups];
    uint32_t mw[kGroups];
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
      const int g = group_of(u);
      if (g < gpr) {
        w[u] = *(const u32x4*)(gr + g * 16);
        mw[u] = ar[g >> 2];
      }
    }
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
      const int g = group_of(u);
      if (g < gpr) {
        const uint32_t bits = mw[u] >> ((g & 3) * 8);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = ((bits >> (2 * q)) & 1u) ? 0x0000ffffu : 0u;
          const uint32_t hi = ((bits >> (2 * q + 1)) & 1u) ? 0xffff0000u : 0u;
          w[u][q] &= lo | hi;  // masked-out elements become +0
        }
        *(u32x4*)(dx + (int64_t)row * lddx * 2 + g * 16) = w[u];
      }
    }
  }
}

// part[blockIdx.y][col] = sum of rows [y*rpb, (y+1)*rpb) of column col, in row order; one
// thread per 8 columns, 8 rows loaded at a time and then added in order
template <int DT>
__global__ void colsum_partial_kernel(const char* x, int64_t ldx, float* part, int M, int N, int rpb) {
  const int col = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (col >= N) return;
  const int64_t r0 = (int64_t)blockIdx.y * rpb;
  const int64_t r1 = r0 + rpb < M ? r0 + rpb : M;
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t rb = r0; rb < r1; rb += 8) {
    u32x4 w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (rb + u < r1) w[u] = *(const u32x4*)(x + ((rb + u) * ldx + col) * 2);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (rb + u < r1) {
        float f[8];
        unpack8<DT>(w[u], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += f[e];
      }
    }
  }
  float* o = part + (int64_t)blockIdx.y * N + col;
  *(f32x4*)o = f32x4{s[0], s[1], s[2], s[3]};
  *(f32x4*)(o + 4) = f32x4{s[4], s[5], s[6], s[7]};
}

// bgrad[n] = sum over t of part[t][n].  One workgroup sums 64 columns; its 256 threads are 16
// row groups x 16 column quads.  Row group g adds the partials t = g, g + 16, g + 32, ... in
// increasing t, with the loads of 8 partials in flight at a time, and the 16 group sums are
// then added in order of g through LDS.  The order is fixed, so a result repeats bit for bit,
// and N / 64 workgroups spread the 4 * nparts * N bytes over the chip (one thread per column
// quad over all partials left most CUs idle and paid one round trip per 8 partials: 47 us for
// 256 x 16384 partials).
// Both sums are compensated (Kahan's summation: each addition's rounding error is carried
// into the next addend), so the result stays within a few float32 roundings of the partials'
// exact sum however many partials there are; plain float32 sums of the 8.4 million partials of
// a 2^31-row matrix, 524288 per row group, drift by about 1e-3 relative.
constexpr int kBgColsPerBlock = 64;
constexpr int kBgGroups = kEwThreads / (kBgColsPerBlock / 4);
// (Once a running sum is infinite or NaN, its compensation is reset to zero: (inf - inf) would
// otherwise turn an infinite sum into NaN, where plain summation keeps the infinity.)
__device__ __forceinline__ void kahan_add(f32x4& s, f32x4& c, f32x4 v) {
  const f32x4 y = v - c;
  const f32x4 t = s + y;
  const f32x4 e = (t - s) - y;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = __builtin_isfinite(t[i]) ? e[i] : 0.0f;
  s = t;
}
__global__ __launch_bounds__(kEwThreads) void bgrad_reduce_kernel(const float* part, int nparts, float* bgrad, int N) {
  __shared__ f32x4 red[kBgGroups][kBgColsPerBlock / 4];
  const int q = threadIdx.x % (kBgColsPerBlock / 4), g = threadIdx.x / (kBgColsPerBlock / 4);
  const int col = blockIdx.x * kBgColsPerBlock + q * 4;
  f32x4 s = {0.f, 0.f, 0.f, 0.f}, c = {0.f, 0.f, 0.f, 0.f};
  if (col < N) {
    for (int t0 = g; t0 < nparts; t0 += kBgGroups * 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (t0 + kBgGroups * u < nparts) v[u] = *(const f32x4*)(part + (int64_t)(t0 + kBgGroups * u) * N + col);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (t0 + kBgGroups * u < nparts) kahan_add(s, c, v[u]);
    }
  }
  red[g][q] = s - c;
  __syncthreads();
  if (g == 0 && col < N) {
    f32x4 r = red[0][q], rc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 1; i < kBgGroups; ++i) kahan_add(r, rc, red[i][q]);
    *(f32x4*)(bgrad + col) = r - rc;
  }
}

__global__ void fill_zero_kernel(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

template <int DT>
__global__ void silu_mul_kernel(const char* g, const char* u, int64_t ldgu, char* h, int64_t ldh, int M, int N) {
  const int gpr = N / 8;
  for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
    const int64_t ro = (int64_t)row * ldgu * 2;
    u32x4 wg[kGroups], wu[kGroups];
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      const int c = group_of(q);
      if (c < gpr) {
        wg[q] = *(const u32x4*)(g + ro + c * 16);
        wu[q] = *(const u32x4*)(u + ro + c * 16);
      }
    }
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      const int c = group_of(q);
      if (c < gpr) {
        float fg[8], fu[8];
        unpack8<DT>(wg[q], fg);
        unpack8<DT>(wu[q], fu);
#pragma unroll
        for (int e = 0; e < 8; ++e) fg[e] = fg[e] * sigmoid_f(fg[e]) * fu[e];
        *(u32x4*)(h + (int64_t)row * ldh * 2 + c * 16) = pack8<DT>(fg);
      }
    }
  }
}

template <int DT>
__global__ void dswiglu_kernel(const char* dh, int64_t lddh, const char* gate, const char* up, int64_t ld_gu,
                               char* dg, int64_t lddg, char* du, int64_t lddu, int M, int N) {
  const int gpr = N / 8;
  for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
    u32x4 wd[kGroups], wg[kGroups], wu[kGroups];
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      const int c = group_of(q);
      if (c < gpr) {
        wd[q] = *(const u32x4*)(dh + (int64_t)row * lddh * 2 + c * 16);
        wg[q] = *(const u32x4*)(gate + (int64_t)row * ld_gu * 2 + c * 16);
        wu[q] = *(const u32x4*)(up + (int64_t)row * ld_gu * 2 + c * 16);
      }
    }
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      const int c = group_of(q);
      if (c < gpr) {
        float fd[8], fg[8], fu[8], og[8], ou[8];
        unpack8<DT>(wd[q], fd);
        unpack8<DT>(wg[q], fg);
        unpack8<DT>(wu[q], fu);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sg = sigmoid_f(fg[e]);
          const float t = fd[e] * sg;
          ou[e] = t * fg[e];
          og[e] = t * fu[e] * (1.0f + fg[e] * (1.0f - sg));
        }
        *(u32x4*)(dg + (int64_t)row * lddg * 2 + c * 16) = pack8<DT>(og);
        *(u32x4*)(du + (int64_t)row * lddu * 2 + c * 16) = pack8<DT>(ou);
      }
    }
  }
}

// unfused GELU forward, in place: aux = z (when aux is given), z = gelu(z)
template <int DT>
__global__ void gelu_apply_kernel(char* z, int64_t ldz, char* aux, int64_t ld_aux, int M, int N) {
  const int gpr = N / 8;
  for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
    char* zr = z + (int64_t)row * ldz * 2;
    u32x4 w[kGroups];
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      const int c = group_of(q);
      if (c < gpr) w[q] = *(const u32x4*)(zr + c * 16);
    }
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      const int c = group_of(q);
      if (c < gpr) {
        if (aux) *(u32x4*)(aux + (int64_t)row * ld_aux * 2 + c * 16) = w[q];
        float f[8];
        unpack8<DT>(w[q], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = gelu_f(f[e]);
        *(u32x4*)(zr + c * 16) = pack8<DT>(f);
      }
    }
  }
}

// unfused GELU backward, in place: g = g * gelu'(aux)
template <int DT>
__global__ void dgelu_apply_kernel(char* g, int64_t ldg, const char* aux, int64_t ld_aux, int M, int N) {
  const int gpr = N / 8;
  for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
    char* gr = g + (int64_t)row * ldg * 2;
    u32x4 wg[kGroups], wa[kGroups];
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      const int c = group_of(q);
      if (c < gpr) {
        wg[q] = *(const u32x4*)(gr + c * 16);
        wa[q] = *(const u32x4*)(aux + (int64_t)row * ld_aux * 2 + c * 16);
      }
    }
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      const int c = group_of(q);
      if (c < gpr) {
        float fg[8], fa[8];
        unpack8<DT>(wg[q], fg);
        unpack8<DT>(wa[q], fa);
#pragma unroll
        for (int e = 0; e < 8; ++e) fg[e] *= gelu_grad_f(fa[e]);
        *(u32x4*)(gr + c * 16) = pack8<DT>(fg);
      }
    }
  }
}

inline int ew_blocks(int64_t work) {
  // grid-stride kernels (fill, bgrad reduction): enough resident waves to saturate HBM
  int64_t b = (work + kEwThreads - 1) / kEwThreads;
  return (int)(b < 2048 ? (b < 1 ? 1 : b) : 2048);
}

// row-tiled grid for `gpr` 8-column groups per row
inline dim3 row_grid(int M, int gpr) {
  const int gx = (gpr + kEwThreads * kGroups - 1) / (kEwThreads * kGroups);
  return dim3(gx < 1 ? 1 : gx, M < 65535 ? (M < 1 ? 1 : M) : 65535);
}

}  // namespace

#define EP_DT_DISPATCH(dt, ...)                 \
  do {                                          \
    if ((dt) == T_F16) {                        \
      constexpr int DTV = T_F16;                \
      __VA_ARGS__;                              \
    } else {                                    \
      constexpr int DTV = T_BF16;               \
      __VA_ARGS__;                              \
    }                                           \
  } while (0)

hipError_t launch_bias_add(int dtype, void* z, int64_t ldz, const void* bias, int M, int N, hipStream_t s) {
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(bias_add_kernel<DTV>, row_grid(M, N / 8), dim3(kEwThreads), 0, s, (char*)z, ldz,
                                           (const char*)bias, M, N));
  return hipGetLastError();
}

hipError_t launch_relu_pack(int dtype, const void* z, int64_t ldz, void* y, int64_t ldy, uint32_t* aux,
                            int64_t ld_aux, int M, int N, int with_mask, hipStream_t s) {
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(relu_pack_kernel<DTV>, row_grid(M, (N + 31) / 32 * 4), dim3(kEwThreads), 0, s, (const char*)z,
                                           ldz, (char*)y, ldy, aux, ld_aux, M, N, with_mask));
  return hipGetLastError();
}

hipError_t launch_mask_apply(int dtype, const void* g, int64_t ldg, const uint32_t* aux, int64_t ld_aux, void* dx,
                             int64_t lddx, int M, int N, hipStream_t s) {
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(mask_apply_kernel<DTV>, row_grid(M, N / 8), dim3(kEwThreads), 0, s,
                                           (const char*)g, ldg, aux, ld_aux, (char*)dx, lddx, M, N));
  return hipGetLastError();
}

hipError_t launch_colsum_partial(int dtype, const void* x, int64_t ldx, float* part, int M, int N, int rpb,
                                 hipStream_t s) {
  const dim3 grid((N / 8 + kEwThreads - 1) / kEwThreads, (unsigned)(((int64_t)M + rpb - 1) / rpb));
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(colsum_partial_kernel<DTV>, grid, dim3(kEwThreads), 0, s,
                                           (const char*)x, ldx, part, M, N, rpb));
  return hipGetLastError();
}

hipError_t launch_bgrad_reduce(const float* part, int nparts, float* bgrad, int N, hipStream_t s) {
  const int nb = (N + kBgColsPerBlock - 1) / kBgColsPerBlock;
  hipLaunchKernelGGL(bgrad_reduce_kernel, dim3(nb), dim3(kEwThreads), 0, s, part, nparts, bgrad, N);
  return hipGetLastError();
}

hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3(ew_blocks(n)), dim3(kEwThreads), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_silu_mul(int dtype, const void* g, const void* u, int64_t ldgu, void* h, int64_t ldh, int M, int N,
                           hipStream_t s) {
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(silu_mul_kernel<DTV>, row_grid(M, N / 8), dim3(kEwThreads), 0, s, (const char*)g,
                                           (const char*)u, ldgu, (char*)h, ldh, M, N));
  return hipGetLastError();
}

hipError_t launch_dswiglu(int dtype, const void* dh, int64_t lddh, const void* gate, const void* up, int64_t ld_gu,
                          void* dg, int64_t lddg, void* du, int64_t lddu, int M, int N, hipStream_t s) {
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(dswiglu_kernel<DTV>, row_grid(M, N / 8), dim3(kEwThreads), 0, s, (const char*)dh,
                                           lddh, (const char*)gate, (const char*)up, ld_gu, (char*)dg, lddg, (char*)du,
                                           lddu, M, N));
  return hipGetLastError();
}

hipError_t launch_gelu_apply(int dtype, void* z, int64_t ldz, void* aux, int64_t ld_aux, int M, int N,
                             hipStream_t s) {
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(gelu_apply_kernel<DTV>, row_grid(M, N / 8), dim3(kEwThreads), 0, s, (char*)z, ldz,
                                           (char*)aux, ld_aux, M, N));
  return hipGetLastError();
}

hipError_t launch_dgelu_apply(int dtype, void* g, int64_t ldg, const void* aux, int64_t ld_aux, int M, int N,
                              hipStream_t s) {
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(dgelu_apply_kernel<DTV>, row_grid(M, N / 8), dim3(kEwThreads), 0, s, (char*)g, ldg,
                                           (const char*)aux, ld_aux, M, N));
  return hipGetLastError();
}

}  // namespace ep
