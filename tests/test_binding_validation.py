"""CPU tests of the Python binding's tensor checks (no GPU work).

The C ABI receives raw pointers and leading dimensions only, so the binding checks every
tensor against the problem before planning: device, dtype, shape and strides.  Each case
below breaks one of them on host tensors and expects a ValueError naming it; a request
that passes every shape and dtype check still fails because host tensors are not on a
HIP device.
"""
import pytest
import torch

from dense_gemm_epilogues_amd import validate_operands

F16 = torch.float16
M, N, K = 64, 80, 48  # N % 32 != 0: the mask rows hold ceil(N/32) = 3 words


def t(*shape, dtype=F16):
    return torch.zeros(*shape, dtype=dtype)


def run(a=None, b=None, epilog="DEFAULT", ins=None, b_layout="KN", a_layout="MK", out=None, aux=None):
    a = t(M, K) if a is None else a
    b = (t(K, N) if b_layout == "KN" else t(N, K)) if b is None else b
    return validate_operands(a, b, epilog, ins or {}, b_layout, a_layout, out, aux or {})


def raises(match, **kw):
    with pytest.raises(ValueError, match=match):
        run(**kw)


def test_valid_host_operands_reach_the_device_check():
    for lay in ("KN", "NK"):
        raises("CUDA", b_layout=lay)
    raises("CUDA", a=t(K, M), a_layout="KM")
    # mask rows may be padded past ceil(N/32) words
    raises("CUDA", epilog="RELU_AUX_BIAS", ins={"bias": t(N)}, aux={"relu_aux": torch.zeros(M, 4, dtype=torch.int32)})
    raises("CUDA", epilog="SWIGLU_AUX", ins={"b2": t(K, N)}, aux={"gu": t(M, 2 * N)})
    raises("CUDA", epilog="DSWIGLU", ins={"gate": t(M, N), "up": t(M, N)}, aux={"d_up": t(M, N)})
    raises("CUDA", epilog="DRELU_BGRAD", ins={"relu_aux": torch.zeros(M, 3, dtype=torch.int32)},
           aux={"drelu_bgrad": t(N, dtype=torch.float32)})
    # column views of a wider buffer (row stride above the row length) are accepted
    wide = t(M, 2 * N)
    raises("CUDA", epilog="DSWIGLU", ins={"gate": wide[:, :N], "up": wide[:, N:]}, out=t(M, 2 * N)[:, :N])


def test_inner_dimension_and_layout():
    raises("b must have shape", b=t(K + 8, N))                 # K x N with the wrong K
    raises("b must have shape", b=t(N, K + 8), b_layout="NK")  # N x K with the wrong K
    raises("unknown b_layout", b_layout="TN")
    raises("unknown a_layout", a_layout="XX")
    raises("must be 2-D", a=t(M, K, 1))


def test_dtypes():
    raises("a must be float16 or bfloat16", a=t(M, K, dtype=torch.float32))
    raises("b must be torch.float16", b=t(K, N, dtype=torch.bfloat16))
    raises("out must be torch.float16", out=t(M, N, dtype=torch.bfloat16))
    raises("bias must be torch.float16", epilog="BIAS", ins={"bias": t(N, dtype=torch.float32)})
    raises("relu_aux must be torch.int32", epilog="DRELU_BGRAD", ins={"relu_aux": t(M, 3, dtype=torch.int16)})
    raises("drelu_bgrad.*float32", epilog="DRELU_BGRAD", ins={"relu_aux": torch.zeros(M, 3, dtype=torch.int32)},
           aux={"drelu_bgrad": t(N)})
    raises("gate must be torch.float16", epilog="DSWIGLU",
           ins={"gate": t(M, N, dtype=torch.bfloat16), "up": t(M, N)})


def test_shapes_of_epilog_tensors():
    raises("bias must be a contiguous", epilog="BIAS", ins={"bias": t(N - 8)})
    raises("bias must be a contiguous", epilog="BIAS", ins={"bias": t(2 * N)[::2]})
    raises("relu_aux must have shape", epilog="DRELU_BGRAD", ins={"relu_aux": torch.zeros(M, 2, dtype=torch.int32)})
    raises("relu_aux.*must have shape", epilog="RELU_AUX_BIAS", ins={"bias": t(N)},
           aux={"relu_aux": torch.zeros(M - 1, 3, dtype=torch.int32)})
    raises("out must have shape", out=t(M, N - 8))
    raises("b2 must have shape", epilog="SWIGLU", ins={"b2": t(K, N - 8)})
    raises("b2 must have the same row stride", epilog="SWIGLU", ins={"b2": t(K, 2 * N)[:, :N]})
    raises("gate and up must share a row stride", epilog="DSWIGLU",
           ins={"gate": t(M, N), "up": t(M, 2 * N)[:, :N]})
    raises("up must have shape", epilog="DSWIGLU", ins={"gate": t(M, N), "up": t(M + 1, N)})
    raises("gelu_aux must have shape", epilog="DGELU_BGRAD", ins={"gelu_aux": t(M, N + 8)})
    raises("gu.*must have shape", epilog="SWIGLU_AUX", ins={"b2": t(K, N)}, aux={"gu": t(M, N)})
    raises("d_up.*must have shape", epilog="DSWIGLU", ins={"gate": t(M, N), "up": t(M, N)}, aux={"d_up": t(M, 8)})
    raises("unit column stride", out=t(N, M).t())


def test_inputs_required_and_extra():
    raises("needs epilog_inputs\\['bias'\\]", epilog="RELU_BIAS")
    raises("needs epilog_inputs\\['up'\\]", epilog="DSWIGLU", ins={"gate": t(M, N)})
    raises("takes no epilog_inputs\\['bias'\\]", epilog="DEFAULT", ins={"bias": t(N)})
    raises("unknown aux_out", aux={"mask": t(M, 3)})
    raises("must be a torch.Tensor", epilog="BIAS", ins={"bias": [0.0] * N})


def test_device_mismatch():
    meta = torch.zeros(M, N, dtype=F16, device="meta")
    raises("is on meta", out=meta)
