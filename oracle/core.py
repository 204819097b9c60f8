"""Plain float64 definitions of every operation the fused kernels compute.

Test infrastructure: only tests, the smoke check and the benchmark's CPU-baseline leg
use this module.  No blocking, fusion or reordering beyond the definitions: each
function is the written-out definition, with numpy's matmul as the one library step.

Conventions (shared with the library's C header only through this prose, not code):
  * A is row-major M x K.  B is either "KN" (row-major K x N, so Z = A B) or "NK"
    (row-major N x K, a torch Linear weight, so Z = A B^T).
  * Outputs are row-major M x N.  Half-precision inputs are decoded exactly to float64
    before any arithmetic; nothing is rounded afterwards.
"""
import numpy as np
from scipy.special import erf as _erf


# ----------------------------------------------------------------------------- decoding
def decode_f16(x):
    """Exact float64 value of IEEE binary16 data (every binary16 is a float64)."""
    return np.asarray(x, dtype=np.float16).astype(np.float64)


def decode_bf16_bits(bits):
    """Exact float64 value of bfloat16 data given as its raw uint16 bit patterns.

    A bfloat16 is the upper half of a binary32: shifting the 16 bits into the high half
    of a uint32 and reinterpreting gives the float32 with the same value.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- GEMM
def matmul(a, b, b_layout):
    """Z = A . B with B given in layout "KN" (K x N) or "NK" (N x K, used as B^T).

    The GEMM that every epilog sits on ("The problem addressed by fused epilogs",
    Fusing Matmul Epilogs with nvmath-python; blog post paragraph 4: half inputs,
    wide accumulation -- here float64, the exact-up-to-rounding-order value).
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if b_layout == "KN":
        bk = b
    elif b_layout == "NK":
        bk = b.T
    else:
        raise ValueError("b_layout must be 'KN' or 'NK'")
    if a.shape[1] != bk.shape[0]:
        raise ValueError(f"inner dimensions differ: {a.shape} vs {bk.shape}")
    return a @ bk


def bias_epilog(a, b, bias, b_layout):
    """BIAS epilog: P = A.B + bias, one bias value per output column (feature).

    Fusing Matmul Epilogs with nvmath-python, "The problem addressed by fused epilogs":
    the bias is added to each output column.  (The blog post's listing declares an
    (m, 1) bias, which is the same computation in the transposed, feature-major
    orientation; with batch-major rows the bias runs along the N features.)
    """
    z = matmul(a, b, b_layout)
    bias = np.asarray(bias, dtype=np.float64).reshape(-1)
    if bias.shape[0] != z.shape[1]:
        raise ValueError("bias length must equal N")
    return z + bias[None, :]


def relu_bias(a, b, bias, b_layout):
    """RELU_BIAS epilog: Y = max(P, 0) with P the BIAS result.

    "Forward-pass capabilities in the source": RELU_BIAS combines the matrix product,
    the bias addition and ReLU.  The predicate is strict (P > 0); where it fails the
    output is +0.
    """
    p = bias_epilog(a, b, bias, b_layout)
    return np.where(p > 0.0, p, 0.0)


# ----------------------------------------------------------------------------- ReLU mask
def pack_relu_mask(pred, ld_aux=None):
    """Pack a boolean M x N predicate into the relu_aux word layout.

    Layout (fixed by this library; the source calls relu_aux an opaque bit-encoded mask
    meant for the matching backward epilog): one bit per element, row-major, 32
    elements per uint32 along the feature dimension.  Bit b of word w in row i is the
    predicate of element (i, 32 w + b); the least significant bit is the lowest column.
    Bits past column N-1 and words past ceil(N/32) (row padding up to ld_aux) are 0.
    """
    pred = np.asarray(pred, dtype=bool)
    m, n = pred.shape
    nw = (n + 31) // 32
    if ld_aux is None:
        ld_aux = nw
    if ld_aux < nw:
        raise ValueError("ld_aux must be at least ceil(N/32)")
    bits = np.zeros((m, nw * 32), dtype=np.uint64)
    bits[:, :n] = pred
    bits = bits.reshape(m, nw, 32)
    weights = np.left_shift(np.uint64(1), np.arange(32, dtype=np.uint64))
    words = np.zeros((m, ld_aux), dtype=np.uint32)
    # a sum of distinct powers of two is their bitwise OR
    words[:, :nw] = (bits * weights[None, None, :]).sum(axis=2).astype(np.uint32)
    return words


def unpack_relu_mask(words, n):
    """Inverse of pack_relu_mask: the M x N boolean mask held in the first N bits."""
    words = np.asarray(words, dtype=np.uint32)
    nw = (n + 31) // 32
    if words.shape[1] < nw:
        raise ValueError("mask rows are shorter than ceil(N/32) words")
    shifts = np.arange(32, dtype=np.uint32)
    bits = (words[:, :nw, None] >> shifts[None, None, :]) & np.uint32(1)
    return bits.reshape(words.shape[0], nw * 32)[:, :n].astype(bool)


def relu_aux_bias(a, b, bias, b_layout, ld_aux=None):
    """RELU_AUX_BIAS epilog: (Y, relu_aux words, P).

    "Forward-pass capabilities in the source": the same forward work as RELU_BIAS, and
    in addition an auxiliary relu_aux output, the bit-encoded ReLU mask that the
    DRELU_BGRAD backward epilog consumes.  The bit is set iff the pre-activation is
    strictly positive, the same predicate ReLU uses, so Y and the mask never disagree.
    P (the float64 pre-activation) is returned so callers can apply the mask tolerance.
    """
    p = bias_epilog(a, b, bias, b_layout)
    pred = p > 0.0
    y = np.where(pred, p, 0.0)
    return y, pack_relu_mask(pred, ld_aux), p


# ----------------------------------------------------------------------------- backward
def drelu_bgrad(a, b, b_layout, relu_aux_in):
    """DRELU_BGRAD epilog: (dX, bgrad).

    "Backward-pass path shown in the example": the product of the output gradient with
    the transposed weight is masked by the relu_aux of the forward pass, and the
    auxiliary output drelu_bgrad is the column-wise sum over the batch of that masked
    product (the bias gradient).  With A = dY (M x N_out) and B = W given as "NK"
    (W is N_in x N_out row-major, i.e. the forward's K x N weight), G = dY W^T.
    The sum is over the unrounded masked values.
    """
    g = matmul(a, b, b_layout)
    mask = unpack_relu_mask(relu_aux_in, g.shape[1])
    dx = np.where(mask, g, 0.0)
    return dx, dx.sum(axis=0)


def bgrad_all_ones_closed_form(a, b, b_layout):
    """bgrad of DRELU_BGRAD when every mask bit is set, without forming the product.

    sum_i (A B)[i, j] = sum_k (sum_i A[i, k]) B[k, j]: the column sums of A times B.
    Costs O(MK + NK), so it checks full-size outputs the direct definition cannot.
    """
    a = np.asarray(a, dtype=np.float64)
    s = a.sum(axis=0)
    b = np.asarray(b, dtype=np.float64)
    if b_layout == "KN":
        return s @ b
    if b_layout == "NK":
        return b @ s
    raise ValueError("b_layout must be 'KN' or 'NK'")


# ----------------------------------------------------------------------------- SwiGLU
def sigmoid(t):
    """Logistic function, evaluated without overflow: 1/(1+e^-t) for t >= 0 and
    e^t/(1+e^t) for t < 0."""
    t = np.asarray(t, dtype=np.float64)
    out = np.empty_like(t)
    pos = t >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-t[pos]))
    e = np.exp(t[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu(t):
    """SiLU(t) = t * sigmoid(t)."""
    t = np.asarray(t, dtype=np.float64)
    return t * sigmoid(t)


def silu_grad(t):
    """d/dt SiLU(t) = s + t s (1 - s) = s (1 + t (1 - s)), s = sigmoid(t)."""
    t = np.asarray(t, dtype=np.float64)
    s = sigmoid(t)
    return s * (1.0 + t * (1.0 - s))


def swiglu(x, wg, wu, b_layout="NK"):
    """SwiGLU forward h = silu(x Wg^T) * (x Wu^T).

    gemm_swiglu_mlp_fusion.py, module docstring: the forward computes silu(x @ Wg^T) *
    (x @ Wu^T), gate GEMM + up GEMM + SiLU + multiply in one kernel; the weights are
    (I, H) Linear weights, hence layout "NK".  Returns (h, g, u) in float64.
    """
    g = matmul(x, wg, b_layout)
    u = matmul(x, wu, b_layout)
    return silu(g) * u, g, u


def dswiglu(dout, wd, gate, up, b_layout="KN"):
    """GEMM + dSwiGLU backward epilog: (d_gate, d_up, dh).

    gemm_swiglu_mlp_fusion.py, module docstring: the backward fuses dSwiGLU as the
    epilogue of matmul(dout, Wd) -> dh, with Wd the (H, I) down-projection weight, so
    dh = dout . Wd (layout "KN").  The derivative of h = silu(g) u gives
        d_gate = dh * u * silu'(g),   d_up = dh * silu(g),
    evaluated at the saved pre-activations gate and up.
    """
    dh = matmul(dout, wd, b_layout)
    gate = np.asarray(gate, dtype=np.float64)
    up = np.asarray(up, dtype=np.float64)
    return dh * up * silu_grad(gate), dh * silu(gate), dh


# ---------------------------------------------------------------------------- GELU
# The hotdry.top cuBLASLt post (its opening paragraph and the paragraph listing the
# predefined epilogs) names GELU as a fusable activation and GELU_BIAS as an epilog but does
# not say which GELU.  The exact form is used: gelu(t) = t * Phi(t), Phi the standard normal
# CDF.  GELU_AUX_BIAS and DGELU_BGRAD follow the RELU_AUX_BIAS / DRELU_BGRAD pair: the forward
# also returns its pre-activation, the backward scales dY W^T by gelu' of that stored
# pre-activation and reduces the result over the batch into the bias gradient.

def gelu(t):
    """t * Phi(t) = t / 2 * (1 + erf(t / sqrt(2)))."""
    t = np.asarray(t, dtype=np.float64)
    return 0.5 * t * (1.0 + _erf(t / np.sqrt(2.0)))


def gelu_grad(t):
    """d gelu / dt = Phi(t) + t * phi(t), phi(t) = exp(-t^2 / 2) / sqrt(2 pi)."""
    t = np.asarray(t, dtype=np.float64)
    return 0.5 * (1.0 + _erf(t / np.sqrt(2.0))) + t * np.exp(-0.5 * t * t) / np.sqrt(2.0 * np.pi)


def gelu_aux_bias(a, b, bias, b_layout):
    """GELU_BIAS / GELU_AUX_BIAS epilog: (Y, P) with P = A B + bias (the pre-activation,
    returned by GELU_AUX_BIAS as its auxiliary output) and Y = gelu(P)."""
    p = bias_epilog(a, b, bias, b_layout)
    return gelu(p), p


def dgelu_bgrad(a, b, b_layout, p_aux):
    """DGELU_BGRAD epilog: (dX, bgrad) with dX = (dY W^T) * gelu'(P) elementwise, P the stored
    pre-activation of the forward (the exact values the GPU consumed), and bgrad the
    column-wise sum over the batch of the unrounded dX."""
    g = matmul(a, b, b_layout)
    dx = g * gelu_grad(p_aux)
    return dx, dx.sum(axis=0)
