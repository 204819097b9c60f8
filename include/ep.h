/*
 * ep.h -- C ABI of the fused GEMM + epilogue library for AMD Instinct MI355X (gfx950).
 *
 * The call sequence mirrors the stateful plan/execute/free split described on the pages:
 *   - "Fusing Matmul Epilogs with nvmath-python", section "The problem addressed by fused
 *     epilogs": a stateful Matmul separates setup and planning from repeated execution;
 *   - the hotdry.top post "nvmath-python wraps cuBLASLt" (paragraphs 3-6): construct with
 *     the operands, plan once with an epilog and its epilog_inputs, execute many times
 *     asynchronously on a stream, free the internal resources at the end.
 *
 * Conventions used by every entry point:
 *   - A is row-major M x K with leading dimension lda (elements).
 *   - B is row-major K x N (EP_B_KN, N contiguous) or row-major N x K (EP_B_NK, K contiguous,
 *     i.e. a torch Linear weight, used as B^T) with leading dimension ldb (elements).
 *   - D is row-major M x N with leading dimension ldd (elements).
 *   - Elements are IEEE binary16 (EP_F16) or bfloat16 (EP_BF16); products are formed
 *     exactly and accumulated in float32; outputs are rounded to the input type with
 *     round-to-nearest-even.
 *   - All pointers are device pointers (hipMalloc / torch CUDA tensors) except the ones
 *     to the ep_* structs and the char buffer of ep_plan_info, which are host pointers.
 *   - Every call returns ep_status; nothing aborts, exits or throws across the ABI.
 *     On any error no output buffer is written. ep_last_error() gives a thread-local
 *     text for the last error of the calling thread.
 *
 * Ownership: the caller owns every tensor (inputs and outputs). The library owns the
 * handle and the workspace it allocates in ep_plan (bias-gradient partial sums, and the
 * intermediates of the unfused baseline path); ep_free releases both.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 3: ep_options.split_tail, ep_execute_noalloc and ep_plan_describe; 2: ep_options.split_k */
#define EP_ABI_VERSION 3

typedef struct ep_plan_s* ep_handle;

typedef enum {
  EP_OK = 0,
  EP_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size or leading dimension */
  EP_ERR_UNSUPPORTED = 2,   /* well-formed request this library does not implement */
  EP_ERR_OUT_OF_MEMORY = 3, /* workspace allocation failed */
  EP_ERR_HIP = 4,           /* a HIP runtime call failed (no device, launch failure) */
  EP_ERR_INTERNAL = 5
} ep_status;

typedef enum { EP_F16 = 0, EP_BF16 = 1 } ep_dtype;

typedef enum { EP_B_KN = 0, EP_B_NK = 1 } ep_b_layout;

/* EP_A_MK (default): A is row-major M x K.  EP_A_KM: A is given row-major K x M (M
 * contiguous, row stride lda >= m) and the GEMM uses its transpose, as the weight gradient
 * of a linear layer needs (dW = X^T dY contracts over the batch).  EP_A_KM requires m % 8 == 0
 * and the DEFAULT epilog. */
typedef enum { EP_A_MK = 0, EP_A_KM = 1 } ep_a_layout;

/*
 * Epilogs.  Each is applied to the float32 accumulator tile inside the GEMM kernel before
 * the single store to HBM.
 *
 * EP_EPILOG_DEFAULT        D = A.B.
 * EP_EPILOG_BIAS           D = A.B + bias, one bias value per output column (feature);
 *                          hotdry.top post, paragraph 7 (BIAS epilog).
 * EP_EPILOG_RELU_BIAS      D = relu(A.B + bias); "Fusing Matmul Epilogs with nvmath-python",
 *                          "Forward-pass capabilities in the source".  relu(v) = v if v > 0
 *                          else +0, evaluated on the float32 value before rounding.
 * EP_EPILOG_RELU_AUX_BIAS  as RELU_BIAS, and also writes relu_aux, the bit-encoded ReLU
 *                          mask (same section): bit (j mod 32) of word (j / 32) in row i is
 *                          1 iff the float32 pre-activation of element (i, j) is > 0; the
 *                          least significant bit is the lowest column; bits past column
 *                          N-1 are 0; words are uint32, row stride ld_aux words.
 * EP_EPILOG_DRELU_BGRAD    D = mask .* (A.B) with mask read from relu_aux_in (same bit
 *                          layout, N bits per row), and bgrad[j] = sum_i D[i][j] summed in
 *                          float32 over the unrounded masked values;  "Backward-pass path
 *                          shown in the example".  Typically A = dY (M x N_out) and B = the
 *                          forward weight W (N_in x N_out row-major) as EP_B_NK, so that
 *                          D = dY W^T has N = N_in columns.
 * EP_EPILOG_SWIGLU         D = silu(A.B) .* (A.B2) with B2 (the up weight) in the same
 *                          layout and leading dimension as B (the gate weight); both
 *                          products are kept in float32 until the single store.
 *                          gemm_swiglu_mlp_fusion.py, module docstring (forward).
 * EP_EPILOG_DSWIGLU        with dh = A.B (float32), s = sigmoid(gate):
 *                          D = d_gate = dh .* up .* s .* (1 + gate .* (1 - s)),
 *                          D2 = d_up = dh .* gate .* s;  gate and up are M x N inputs in
 *                          the element type (row stride ld_gu).  gemm_swiglu_mlp_fusion.py,
 *                          module docstring (backward dSwiGLU as a matmul epilogue).
 * EP_EPILOG_SWIGLU_AUX     as SWIGLU, and also writes the two pre-activations to d2 (M x 2N,
 *                          row stride ldd2 >= 2N): columns [0, N) = A.B (gate), [N, 2N) =
 *                          A.B2 (up), rounded to the element type; the layout DSWIGLU reads
 *                          with gate = d2, up = d2 + N, ld_gu = ldd2 (save instead of
 *                          recompute for the backward; gemm_swiglu_mlp_fusion.py docstring).
 * EP_EPILOG_GELU_BIAS      D = gelu(A.B + bias) with the exact GELU, gelu(t) = t Phi(t) =
 *                          t/2 (1 + erf(t / sqrt 2)) (hotdry.top post: GELU_BIAS among the
 *                          predefined epilogs; the post does not fix the GELU variant).
 * EP_EPILOG_GELU_AUX_BIAS  as GELU_BIAS, and also writes gelu_aux = A.B + bias, the
 *                          pre-activation rounded to the element type (M x N, row stride
 *                          ld_gelu_aux), for the backward.
 * EP_EPILOG_DGELU_BGRAD    D = (A.B) .* gelu'(P) with P read from gelu_aux (M x N, element
 *                          type), gelu'(t) = Phi(t) + t phi(t), and bgrad[j] = sum_i D[i][j]
 *                          in float32 over the unrounded values, as DRELU_BGRAD.
 */
typedef enum {
  EP_EPILOG_DEFAULT = 0,
  EP_EPILOG_BIAS = 1,
  EP_EPILOG_RELU_BIAS = 2,
  EP_EPILOG_RELU_AUX_BIAS = 3,
  EP_EPILOG_DRELU_BGRAD = 4,
  EP_EPILOG_SWIGLU = 5,
  EP_EPILOG_DSWIGLU = 6,
  EP_EPILOG_GELU_BIAS = 7,
  EP_EPILOG_GELU_AUX_BIAS = 8,
  EP_EPILOG_DGELU_BGRAD = 9,
  EP_EPILOG_SWIGLU_AUX = 10
} ep_epilog;

/* The GEMM operands, bound at plan time. Sizes and leading dimensions are in elements. */
typedef struct {
  int64_t m, n, k;        /* 1 <= m, n, k < 2^31; n and k multiples of 8 */
  ep_b_layout b_layout;
  const void* a;          /* M x K, lda >= k (EP_A_KM: K x M, lda >= m) */
  int64_t lda;
  const void* b;          /* K x N (ldb >= n) or N x K (ldb >= k) */
  int64_t ldb;
  void* d;                /* M x N output, ldd >= n */
  int64_t ldd;
  ep_a_layout a_layout;   /* EP_A_MK (0) unless the transpose of a K x M A is wanted */
} ep_shape;

/* Epilog inputs and auxiliary outputs (the epilog_inputs dictionary and the aux dictionary
 * of the pages).  Fields an epilog does not use must be NULL / 0. */
typedef struct {
  const void* bias;            /* BIAS, RELU_BIAS, RELU_AUX_BIAS: n elements, input dtype */
  uint32_t* relu_aux;          /* RELU_AUX_BIAS output: m rows of ld_aux words */
  const uint32_t* relu_aux_in; /* DRELU_BGRAD input: m rows of ld_aux words */
  int64_t ld_aux;              /* words per mask row; 0 means ceil(n/32) */
  float* bgrad;                /* DRELU_BGRAD / DGELU_BGRAD output: n floats */
  const void* b2;              /* SWIGLU: the up weight, same layout/ldb as b */
  const void* gate;            /* DSWIGLU inputs: m x n, row stride ld_gu */
  const void* up;
  int64_t ld_gu;               /* 0 means n */
  void* d2;                    /* DSWIGLU output d_up: m x n, row stride ldd2 (0 means ldd);
                                  SWIGLU_AUX output [gate | up]: m x 2n, row stride ldd2
                                  (0 means 2n) */
  int64_t ldd2;
  void* gelu_aux;              /* GELU_AUX_BIAS output / DGELU_BGRAD input: the pre-activation,
                                  m x n in the element type, row stride ld_gelu_aux */
  int64_t ld_gelu_aux;         /* 0 means n */
} ep_epilog_io;

typedef enum { EP_PATH_FUSED = 0, EP_PATH_UNFUSED = 1 } ep_path;
typedef enum { EP_BGRAD_TWO_PASS = 0, EP_BGRAD_ATOMIC = 1 } ep_bgrad_mode;

typedef struct {
  ep_path path;            /* EP_PATH_UNFUSED runs the same GEMM core with the DEFAULT
                              epilog followed by separate elementwise / reduction kernels
                              through HBM intermediates (the baseline fusion is measured
                              against); results agree with the fused path to rounding */
  ep_bgrad_mode bgrad_mode;/* DRELU_BGRAD: deterministic two-pass reduction (default) or
                              float32 atomics into bgrad (order-dependent rounding) */
  int tile_cfg;            /* -1 = choose by shape; otherwise an index < ep_num_tile_cfgs().
                              Configurations 11 and 12 (256x256 tiles, 64-deep k-steps, 16x16
                              MFMAs; 12 with a second barrier per k-step where B is K x N too)
                              need k % 64 == 0 (EP_ERR_UNSUPPORTED otherwise); one of them is
                              the choice by shape for 256x256 tiles whenever k allows it */
  int split_k;             /* fused path: 0 = chosen by shape (split only when the output tiles
                              leave CUs idle); 1 = never; 2..EP_MAX_SPLIT_K = split the K range of
                              every tile into that many parts, each computed by its own
                              workgroup into fp32 partials that a second launch sums (in a fixed
                              order) before running the epilog.  Must be 0 or 1 for the unfused
                              path. */
  int split_tail;          /* with split_k >= 2: 0 = split every tile; 1 = split only the tiles
                              of the last, partly filled round of workgroups (tiles beyond the
                              largest multiple of the resident workgroup slots, fewer than one
                              round), while the others run their whole K range in a launch of
                              their own before them.  Ignored with split_k 0 (the shape model
                              picks both) and 1.  EP_ERR_UNSUPPORTED when the tiles fill whole
                              rounds or less than one. */
  int autotune;            /* fused path, tile_cfg -1 and split_k 0 only: 1 = ep_plan times every
                              allowed (tile configuration, split) pair on the bound buffers and
                              keeps the one with the lowest median of 5 executes (candidates
                              timed in turn, round by round, each execute after a 512 MiB
                              scratch buffer was overwritten so that caches start cold).  The
                              buffers' contents are overwritten, every candidate's workspace
                              and the scratch buffer are allocated at once (temporarily), and
                              ep_plan synchronizes the device.  The choice is cached per
                              (m, n, k, leading dimensions, layout, dtype, epilog) for the
                              process, so later plans of the same problem do not time again.
                              0 = choose by the shape model (default). */
} ep_options;

#define EP_MAX_SPLIT_K 8

/*
 * ep_plan: validate the request, pick a tile configuration, allocate the workspace and
 * bind all pointers.  Checks, in order, before any HIP call: non-null handle out-pointer
 * and shape; 1 <= m, n < 2^31 and 1 <= k <= 2^31 - 64; n % 8 == 0 and k % 8 == 0; the
 * pointers the epilog needs are non-null and the ones it does not use are null; a, b, b2, d,
 * d2, bias, gate, up are 16-byte aligned and relu_aux/relu_aux_in/bgrad 4-byte aligned; every
 * leading dimension is
 * a multiple of 8 elements, at least the row length and below 2^22; ld_aux >= ceil(n/32).
 * A plan whose GEMM grid would need 2^32 or more threads in one launch (for instance m near
 * 2^31 with a 128-row tile configuration) is EP_ERR_UNSUPPORTED.
 * Returns EP_ERR_INVALID_ARG or EP_ERR_UNSUPPORTED on a failed check and EP_ERR_HIP when no
 * HIP device is usable.  On success *out is a new handle, otherwise *out is set to NULL.
 */
ep_status ep_plan(const ep_shape* shape, ep_dtype dtype, ep_epilog epilog,
                  const ep_epilog_io* io, ep_handle* out);

/* ep_plan with options (opt may be NULL for the defaults {FUSED, TWO_PASS, -1, 0, 0}). */
ep_status ep_plan_ex(const ep_shape* shape, ep_dtype dtype, ep_epilog epilog,
                     const ep_epilog_io* io, const ep_options* opt, ep_handle* out);

/*
 * ep_execute: enqueue the planned computation on `stream` (a hipStream_t; NULL = the null
 * stream of the calling thread's current device) and return without synchronizing.  Checks
 * only the handle and that the stream's device is the one the plan was made on; no
 * allocation.  A handle may be executed any number of times, on any stream of its device,
 * but not concurrently on two streams (they would share its workspace).  Returns
 * EP_ERR_INVALID_ARG for a NULL or freed handle or a stream of another device (nothing is
 * launched) and EP_ERR_HIP if a launch fails.
 */
ep_status ep_execute(ep_handle h, void* stream);

/*
 * ep_execute_noalloc: for callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Plans the request exactly as
 * ep_plan_ex does (same checks, statuses and tile choice) and enqueues it on `stream` as
 * ep_execute does, in one call, without any allocation: no plan handle is created, and the
 * workspace (the two-pass bias-gradient partials, the split-K partial tiles) is a static device
 * array of EP_NOALLOC_SCRATCH_BYTES that each GPU holds for the life of the process.
 *   - fused path only (EP_ERR_UNSUPPORTED for EP_PATH_UNFUSED); autotune is EP_ERR_INVALID_ARG;
 *   - a split-K count chosen by shape is reduced until its partials fit the scratch; a request
 *     whose workspace still exceeds it (an explicit split_k, or two-pass bias-gradient
 *     partials -- n floats per row of output tiles, ceil(m/256) rows for the 256-row tiles --
 *     beyond it) is EP_ERR_UNSUPPORTED, with the sizes in ep_last_error;
 *   - `stream` (NULL = null stream) must belong to the calling thread's current device
 *     (EP_ERR_INVALID_ARG otherwise);
 *   - every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (two
 *     streams, or two threads) race and may produce wrong bias gradients or split results;
 *     calls on one stream are ordered and safe.  The scratch keeps the last call's contents;
 *     each call writes every partial it reads.
 * The caller owns every tensor, as with ep_plan.  The first call on a device looks up the
 * scratch's device address (hipGetSymbolAddress) and the device's properties once.
 */
#define EP_NOALLOC_SCRATCH_BYTES (64u << 20)
ep_status ep_execute_noalloc(const ep_shape* shape, ep_dtype dtype, ep_epilog epilog,
                             const ep_epilog_io* io, const ep_options* opt, void* stream);

/* ep_free: release the handle and its workspace.  ep_free(NULL) is EP_OK. The caller must
 * make sure no execution of the handle is still running. */
ep_status ep_free(ep_handle h);

/* Human-readable name of a status code (static storage). */
const char* ep_status_string(ep_status s);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* ep_last_error(void);

/* Writes a NUL-terminated description (tile configuration, grid, workspace bytes, kernel
 * names) into buf[0..n-1]; truncates to fit. */
ep_status ep_plan_info(ep_handle h, char* buf, size_t n);

/* ep_plan_describe: the plan ep_plan_ex would make for these arguments on a device with `cus`
 * compute units, written into buf[0..n-1] as ep_plan_info writes a plan's description
 * (tile configuration, grid, splits, workspace bytes, kernels).  It makes no HIP call and
 * allocates nothing: the arguments are validated as ep_plan_ex validates them (so operand
 * pointers must be non-null and 16-byte aligned where ep_plan_ex requires it), but no pointer
 * is dereferenced.  For capacity planning, and for checking the planner's choices on a host
 * without a GPU (the plan/execute split of "Fusing Matmul Epilogs with nvmath-python", "The
 * problem addressed by fused epilogs": the planning step alone).  Errors: those of
 * ep_plan_ex's validation; EP_ERR_INVALID_ARG if buf is NULL, n is 0, cus is not in
 * 1..65536 or opt->autotune is set (autotuning times kernels on the device). */
ep_status ep_plan_describe(const ep_shape* shape, ep_dtype dtype, ep_epilog epilog, const ep_epilog_io* io,
                           const ep_options* opt, int cus, char* buf, size_t n);

/* Number of selectable tile configurations (valid ep_options.tile_cfg values). */
int ep_num_tile_cfgs(void);

/* EP_ABI_VERSION of the library. */
int ep_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* EP_H */
