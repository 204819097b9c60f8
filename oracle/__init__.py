"""CPU oracle for the fused GEMM + epilogue library (test infrastructure only).

This package is the slow, plain, obviously-correct reference that the HIP kernels are
checked against.  It is evaluated in float64 with numpy on the exact half-precision
values the GPU consumed.  It shares no code with the HIP path and never imports it.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it; the product path (the C library and its Python binding) never does.

Sources, by page:
  * "Fusing Matmul Epilogs with nvmath-python" (nvmath-python epilog summary):
    sections "The problem addressed by fused epilogs", "Forward-pass capabilities in the
    source", "Backward-pass path shown in the example".
  * "nvmath-python wraps cuBLASLt: low-overhead matmul + bias fusion primitives for
    PyTorch" (hotdry.top blog post, paragraphs 3-7 and their listings).
  * "gemm_swiglu_mlp_fusion.py" (cudnn-frontend sample, module docstring and _demo).
  * GELU: named (not defined) by the hotdry.top post; the exact erf form is used.

Every function is pinned by a CPU test (exact rational brute force, closed forms,
invariants, hand-derived fixtures under tests/golden/).  Nothing here is "parity
unpinned".
"""
from .core import (
    decode_f16, decode_bf16_bits, matmul, bias_epilog, relu_bias, relu_aux_bias,
    pack_relu_mask, unpack_relu_mask, drelu_bgrad, bgrad_all_ones_closed_form,
    sigmoid, silu, silu_grad, swiglu, dswiglu, gelu, gelu_grad, gelu_aux_bias, dgelu_bgrad,
)
from .compare import rel_l2, check_half_output, check_mask, check_bgrad, TOL
from .sampling import sample_tiles, sample_columns

__all__ = [
    "decode_f16", "decode_bf16_bits", "matmul", "bias_epilog", "relu_bias", "relu_aux_bias",
    "pack_relu_mask", "unpack_relu_mask", "drelu_bgrad", "bgrad_all_ones_closed_form",
    "sigmoid", "silu", "silu_grad", "swiglu", "dswiglu", "gelu", "gelu_grad", "gelu_aux_bias", "dgelu_bgrad",
    "rel_l2", "check_half_output", "check_mask", "check_bgrad", "TOL",
    "sample_tiles", "sample_columns",
]
