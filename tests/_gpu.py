"""Helpers shared by the GPU parity tests: device checks, decoding, oracle comparison."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def have_gpu():
    try:
        return torch.cuda.is_available() and torch.cuda.device_count() > 0
    except Exception:
        return False


def require_gpu():
    if not have_gpu():
        pytest.skip("no GPU")


def f64(t):
    """float64 numpy copy of a torch fp16/bf16/fp32 tensor, decoded exactly."""
    a = workloads.to_numpy(t)
    if t.dtype == torch.float16:
        return oracle.decode_f16(a)
    if t.dtype == torch.bfloat16:
        return oracle.decode_bf16_bits(a)
    return np.asarray(a, dtype=np.float64)


def words(t):
    return workloads.to_numpy(t).astype(np.uint32)


def assert_half(got, ref, what):
    ok, info = oracle.check_half_output(got, ref)
    assert ok, f"{what}: {info}"
    return info


def assert_mask(got_words, p_ref, what):
    ok, info = oracle.check_mask(got_words, p_ref)
    assert ok, f"{what}: {info}"
    return info


def assert_bgrad(got, ref, what):
    ok, info = oracle.check_bgrad(got, ref)
    assert ok, f"{what}: {info}"
    return info


def say(msg):
    print(msg, flush=True)
