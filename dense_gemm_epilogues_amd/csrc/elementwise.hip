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

// groups of 8 consecutive columns; N % 8 == 0
template <int DT>
__global__ void bias_add_kernel(char* z, int64_t ldz, const char* bias, int M, int N) {
  const int gpr = N / 8;
  const int64_t total = (int64_t)M * gpr;
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = g / gpr;
    const int col = (int)(g - row * gpr) * 8;
    u32x4* p = (u32x4*)(z + (row * ldz + col) * 2);
    float f[8], b[8];
    unpack8<DT>(*p, f);
    unpack8<DT>(*(const u32x4*)(bias + (int64_t)col * 2), b);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] += b[e];
    *p = pack8<DT>(f);
  }
}

// Y = relu(Z); with_mask: also the relu_aux words.  One thread per 8 columns; the 4 threads
// of a 32-column word combine their bytes with lane shuffles.  Block = 256 threads, and a
// row's groups are laid out so that a word's 4 threads are consecutive lanes.
template <int DT>
__global__ void relu_pack_kernel(const char* z, int64_t ldz, char* y, int64_t ldy, uint32_t* aux,
                                 int64_t ld_aux, int M, int N, int with_mask) {
  const int nw = (N + 31) / 32;
  const int gpr = nw * 4;  // 8-column groups per row, padded to whole words
  const int64_t total = (int64_t)M * gpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;  // multiple of 4
  for (int64_t g0 = blockIdx.x * (int64_t)blockDim.x; g0 < total; g0 += stride) {
    const int64_t g = g0 + threadIdx.x;
    const bool valid = g < total;
    const int64_t row = valid ? g / gpr : 0;
    const int col = valid ? (int)(g - row * gpr) * 8 : N;
    uint32_t byte = 0;
    if (valid && col < N) {
      float f[8];
      unpack8<DT>(*(const u32x4*)(z + (row * ldz + col) * 2), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool pr = f[e] > 0.0f;
        byte |= (pr ? 1u : 0u) << e;
        f[e] = pr ? f[e] : 0.0f;
      }
      *(u32x4*)(y + (row * ldy + col) * 2) = pack8<DT>(f);
    }
    if (with_mask) {
      uint32_t w = byte << (8 * (threadIdx.x & 3));
      w |= (uint32_t)__shfl_xor((int)w, 1);
      w |= (uint32_t)__shfl_xor((int)w, 2);
      if (valid && (threadIdx.x & 3) == 0) aux[row * ld_aux + (col >> 5)] = w;
    }
  }
}

template <int DT>
__global__ void mask_apply_kernel(const char* gsrc, int64_t ldg, const uint32_t* aux, int64_t ld_aux,
                                  char* dx, int64_t lddx, int M, int N) {
  const int gpr = N / 8;
  const int64_t total = (int64_t)M * gpr;
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = g / gpr;
    const int col = (int)(g - row * gpr) * 8;
    const uint32_t bits = aux[row * ld_aux + (col >> 5)] >> (col & 31);
    u32x4 w = *(const u32x4*)(gsrc + (row * ldg + col) * 2);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = ((bits >> (2 * q)) & 1u) ? 0x0000ffffu : 0u;
      const uint32_t hi = ((bits >> (2 * q + 1)) & 1u) ? 0xffff0000u : 0u;
      w[q] &= lo | hi;  // masked-out elements become +0
    }
    *(u32x4*)(dx + (row * lddx + col) * 2) = w;
  }
}

// part[blockIdx.y][col] = sum of rows [y*rpb, (y+1)*rpb) of column col; one thread per 8 cols
template <int DT>
__global__ void colsum_partial_kernel(const char* x, int64_t ldx, float* part, int M, int N, int rpb) {
  const int col = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (col >= N) return;
  const int r0 = blockIdx.y * rpb;
  const int r1 = min(M, r0 + rpb);
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = r0; r < r1; ++r) {
    float f[8];
    unpack8<DT>(*(const u32x4*)(x + ((int64_t)r * ldx + col) * 2), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += f[e];
  }
  float* o = part + (int64_t)blockIdx.y * N + col;
  *(f32x4*)o = f32x4{s[0], s[1], s[2], s[3]};
  *(f32x4*)(o + 4) = f32x4{s[4], s[5], s[6], s[7]};
}

// bgrad[n] = sum_t part[t][n], in order of t (deterministic).  The loads of 8 partials are
// issued together and then added in order, so the latency of one round trip is paid per 8
// partials instead of per partial.
__global__ void bgrad_reduce_kernel(const float* part, int nparts, float* bgrad, int N) {
  const int col = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (col >= N) return;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int t0 = 0; t0 < nparts; t0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (t0 + u < nparts) v[u] = *(const f32x4*)(part + (int64_t)(t0 + u) * N + col);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (t0 + u < nparts) s += v[u];
  }
  *(f32x4*)(bgrad + col) = s;
}

__global__ void fill_zero_kernel(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

template <int DT>
__global__ void silu_mul_kernel(const char* g, const char* u, int64_t ldgu, char* h, int64_t ldh, int M, int N) {
  const int gpr = N / 8;
  const int64_t total = (int64_t)M * gpr;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / gpr;
    const int col = (int)(i - row * gpr) * 8;
    float fg[8], fu[8];
    unpack8<DT>(*(const u32x4*)(g + (row * ldgu + col) * 2), fg);
    unpack8<DT>(*(const u32x4*)(u + (row * ldgu + col) * 2), fu);
#pragma unroll
    for (int e = 0; e < 8; ++e) fg[e] = fg[e] * sigmoid_f(fg[e]) * fu[e];
    *(u32x4*)(h + (row * ldh + col) * 2) = pack8<DT>(fg);
  }
}

template <int DT>
__global__ void dswiglu_kernel(const char* dh, int64_t lddh, const char* gate, const char* up, int64_t ld_gu,
                               char* dg, int64_t lddg, char* du, int64_t lddu, int M, int N) {
  const int gpr = N / 8;
  const int64_t total = (int64_t)M * gpr;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / gpr;
    const int col = (int)(i - row * gpr) * 8;
    float fd[8], fg[8], fu[8], og[8], ou[8];
    unpack8<DT>(*(const u32x4*)(dh + (row * lddh + col) * 2), fd);
    unpack8<DT>(*(const u32x4*)(gate + (row * ld_gu + col) * 2), fg);
    unpack8<DT>(*(const u32x4*)(up + (row * ld_gu + col) * 2), fu);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float s = sigmoid_f(fg[e]);
      const float t = fd[e] * s;
      ou[e] = t * fg[e];
      og[e] = t * fu[e] * (1.0f + fg[e] * (1.0f - s));
    }
    *(u32x4*)(dg + (row * lddg + col) * 2) = pack8<DT>(og);
    *(u32x4*)(du + (row * lddu + col) * 2) = pack8<DT>(ou);
  }
}


// unfused GELU forward, in place: aux = z (when aux is given), z = gelu(z)
template <int DT>
__global__ void gelu_apply_kernel(char* z, int64_t ldz, char* aux, int64_t ld_aux, int M, int N) {
  const int gpr = N / 8;
  const int64_t total = (int64_t)M * gpr;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / gpr;
    const int col = (int)(i - row * gpr) * 8;
    const u32x4 raw = *(const u32x4*)(z + (row * ldz + col) * 2);
    if (aux) *(u32x4*)(aux + (row * ld_aux + col) * 2) = raw;
    float f[8];
    unpack8<DT>(raw, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = gelu_f(f[e]);
    *(u32x4*)(z + (row * ldz + col) * 2) = pack8<DT>(f);
  }
}

// unfused GELU backward, in place: g = g * gelu'(aux)
template <int DT>
__global__ void dgelu_apply_kernel(char* g, int64_t ldg, const char* aux, int64_t ld_aux, int M, int N) {
  const int gpr = N / 8;
  const int64_t total = (int64_t)M * gpr;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / gpr;
    const int col = (int)(i - row * gpr) * 8;
    float fg[8], fa[8];
    unpack8<DT>(*(const u32x4*)(g + (row * ldg + col) * 2), fg);
    unpack8<DT>(*(const u32x4*)(aux + (row * ld_aux + col) * 2), fa);
#pragma unroll
    for (int e = 0; e < 8; ++e) fg[e] *= gelu_grad_f(fa[e]);
    *(u32x4*)(g + (row * ldg + col) * 2) = pack8<DT>(fg);
  }
}

constexpr int kEwThreads = 256;

inline int ew_blocks(int64_t work) {
  // enough resident waves to saturate HBM (256 CUs x 8 blocks), capped by the work
  int64_t b = (work + kEwThreads - 1) / kEwThreads;
  return (int)(b < 2048 ? (b < 1 ? 1 : b) : 2048);
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
  const int nb = ew_blocks((int64_t)M * (N / 8));
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(bias_add_kernel<DTV>, dim3(nb), dim3(kEwThreads), 0, s, (char*)z, ldz,
                                           (const char*)bias, M, N));
  return hipGetLastError();
}

hipError_t launch_relu_pack(int dtype, const void* z, int64_t ldz, void* y, int64_t ldy, uint32_t* aux,
                            int64_t ld_aux, int M, int N, int with_mask, hipStream_t s) {
  const int nb = ew_blocks((int64_t)M * ((N + 31) / 32) * 4);
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(relu_pack_kernel<DTV>, dim3(nb), dim3(kEwThreads), 0, s, (const char*)z,
                                           ldz, (char*)y, ldy, aux, ld_aux, M, N, with_mask));
  return hipGetLastError();
}

hipError_t launch_mask_apply(int dtype, const void* g, int64_t ldg, const uint32_t* aux, int64_t ld_aux, void* dx,
                             int64_t lddx, int M, int N, hipStream_t s) {
  const int nb = ew_blocks((int64_t)M * (N / 8));
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(mask_apply_kernel<DTV>, dim3(nb), dim3(kEwThreads), 0, s,
                                           (const char*)g, ldg, aux, ld_aux, (char*)dx, lddx, M, N));
  return hipGetLastError();
}

hipError_t launch_colsum_partial(int dtype, const void* x, int64_t ldx, float* part, int M, int N, int rpb,
                                 hipStream_t s) {
  const dim3 grid((N / 8 + kEwThreads - 1) / kEwThreads, (M + rpb - 1) / rpb);
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(colsum_partial_kernel<DTV>, grid, dim3(kEwThreads), 0, s,
                                           (const char*)x, ldx, part, M, N, rpb));
  return hipGetLastError();
}

hipError_t launch_bgrad_reduce(const float* part, int nparts, float* bgrad, int N, hipStream_t s) {
  const int nb = (N / 4 + kEwThreads - 1) / kEwThreads;
  hipLaunchKernelGGL(bgrad_reduce_kernel, dim3(nb), dim3(kEwThreads), 0, s, part, nparts, bgrad, N);
  return hipGetLastError();
}

hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3(ew_blocks(n)), dim3(kEwThreads), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_silu_mul(int dtype, const void* g, const void* u, int64_t ldgu, void* h, int64_t ldh, int M, int N,
                           hipStream_t s) {
  const int nb = ew_blocks((int64_t)M * (N / 8));
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(silu_mul_kernel<DTV>, dim3(nb), dim3(kEwThreads), 0, s, (const char*)g,
                                           (const char*)u, ldgu, (char*)h, ldh, M, N));
  return hipGetLastError();
}

hipError_t launch_dswiglu(int dtype, const void* dh, int64_t lddh, const void* gate, const void* up, int64_t ld_gu,
                          void* dg, int64_t lddg, void* du, int64_t lddu, int M, int N, hipStream_t s) {
  const int nb = ew_blocks((int64_t)M * (N / 8));
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(dswiglu_kernel<DTV>, dim3(nb), dim3(kEwThreads), 0, s, (const char*)dh,
                                           lddh, (const char*)gate, (const char*)up, ld_gu, (char*)dg, lddg, (char*)du,
                                           lddu, M, N));
  return hipGetLastError();
}

hipError_t launch_gelu_apply(int dtype, void* z, int64_t ldz, void* aux, int64_t ld_aux, int M, int N,
                             hipStream_t s) {
  const int nb = ew_blocks((int64_t)M * (N / 8));
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(gelu_apply_kernel<DTV>, dim3(nb), dim3(kEwThreads), 0, s, (char*)z, ldz,
                                           (char*)aux, ld_aux, M, N));
  return hipGetLastError();
}

hipError_t launch_dgelu_apply(int dtype, void* g, int64_t ldg, const void* aux, int64_t ld_aux, int M, int N,
                              hipStream_t s) {
  const int nb = ew_blocks((int64_t)M * (N / 8));
  EP_DT_DISPATCH(dtype, hipLaunchKernelGGL(dgelu_apply_kernel<DTV>, dim3(nb), dim3(kEwThreads), 0, s, (char*)g, ldg,
                                           (const char*)aux, ld_aux, M, N));
  return hipGetLastError();
}

}  // namespace ep
