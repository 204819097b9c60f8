"""Host-side tests of the C ABI (no GPU work): symbols, status strings and validation.

Every invalid request must be rejected by ep_plan with the documented status before any
HIP call, so these run on a machine without a GPU.  Pointers are fake but aligned
addresses; a rejected plan never dereferences them.
"""
import ctypes
import os
import re

import pytest

import dense_gemm_epilogues_amd as ep
from dense_gemm_epilogues_amd import ep_epilog_io, ep_options, ep_shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")

OK, INVALID, UNSUPPORTED, OOM, HIP, INTERNAL = 0, 1, 2, 3, 4, 5
F16, BF16 = 0, 1
KN, NK = 0, 1
E = ep.EPILOGS

A_PTR, B_PTR, D_PTR, X_PTR = 0x10000, 0x20000, 0x30000, 0x40000


@pytest.fixture(scope="module")
def L():
    return ep.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:ep_status|int|const char\*)\s+(ep_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), f"libep.so does not export {n}"


def test_abi_version_and_status_strings(L):
    assert L.ep_abi_version() == 3
    from tests.test_parity_small_gpu import NUM_TILE_CFGS
    assert L.ep_num_tile_cfgs() == NUM_TILE_CFGS
    for code, name in ep.STATUS.items():
        assert L.ep_status_string(code).decode() == name
    assert L.ep_status_string(99).decode() == "EP_ERR_UNKNOWN"


def test_free_null_and_execute_null(L):
    assert L.ep_free(None) == OK
    assert L.ep_execute(None, None) == INVALID
    assert "handle" in L.ep_last_error().decode()
    buf = ctypes.create_string_buffer(64)
    assert L.ep_plan_info(None, buf, 64) == INVALID


def shape(m=64, n=64, k=64, lay=KN, a=A_PTR, b=B_PTR, d=D_PTR, lda=None, ldb=None, ldd=None, alay=0):
    return ep_shape(m=m, n=n, k=k, b_layout=lay, a=a, lda=(m if alay else k) if lda is None else lda, b=b,
                    ldb=(n if lay == KN else k) if ldb is None else ldb, d=d, ldd=n if ldd is None else ldd,
                    a_layout=alay)


def plan(L, s, epi=E["DEFAULT"], io=None, dtype=F16, opt=None, out=True):
    io = io or ep_epilog_io()
    h = ctypes.c_void_p(0x1234)
    r = L.ep_plan_ex(ctypes.byref(s) if s is not None else None, dtype, epi,
                     ctypes.byref(io) if io is not None else None,
                     ctypes.byref(opt) if opt is not None else None,
                     ctypes.byref(h) if out else None)
    if out and r != OK:
        assert h.value is None, "out handle must be NULL after a failed plan"
    return r, h


CASES = [
    ("null shape", lambda L: plan(L, None)[0], INVALID),
    ("m = 0", lambda L: plan(L, shape(m=0))[0], INVALID),
    ("k < 0", lambda L: plan(L, shape(k=-8))[0], INVALID),
    ("n not multiple of 8", lambda L: plan(L, shape(n=60, ldd=64, ldb=64))[0], UNSUPPORTED),
    ("k not multiple of 8", lambda L: plan(L, shape(k=60, lda=64))[0], UNSUPPORTED),
    ("m >= 2^31", lambda L: plan(L, shape(m=1 << 31))[0], UNSUPPORTED),
    ("k > 2^31 - 64", lambda L: plan(L, shape(k=(1 << 31) - 56))[0], UNSUPPORTED),
    ("unknown dtype", lambda L: plan(L, shape(), dtype=7)[0], UNSUPPORTED),
    ("unknown epilog", lambda L: plan(L, shape(), epi=11)[0], UNSUPPORTED),
    ("SWIGLU_AUX without d2", lambda L: plan(L, shape(lay=NK), E["SWIGLU_AUX"], ep_epilog_io(b2=X_PTR))[0], INVALID),
    ("SWIGLU_AUX ldd2 below 2n", lambda L: plan(L, shape(lay=NK), E["SWIGLU_AUX"],
                                                ep_epilog_io(b2=X_PTR, d2=X_PTR + 8192, ldd2=64))[0], INVALID),
    ("SWIGLU with a stray d2", lambda L: plan(L, shape(lay=NK), E["SWIGLU"], ep_epilog_io(b2=X_PTR, d2=X_PTR + 8192))[0],
     INVALID),
    ("unknown layout", lambda L: plan(L, shape(lay=3))[0], UNSUPPORTED),
    ("null a", lambda L: plan(L, shape(a=0))[0], INVALID),
    ("misaligned b", lambda L: plan(L, shape(b=B_PTR + 8))[0], INVALID),
    ("lda < k", lambda L: plan(L, shape(lda=56))[0], INVALID),
    ("lda not multiple of 8", lambda L: plan(L, shape(lda=68))[0], INVALID),
    ("ldb < n for KN", lambda L: plan(L, shape(ldb=56))[0], INVALID),
    ("ldb < k for NK", lambda L: plan(L, shape(lay=NK, ldb=56))[0], INVALID),
    ("ldd < n", lambda L: plan(L, shape(ldd=56))[0], INVALID),
    ("ld >= 2^22", lambda L: plan(L, shape(lda=1 << 22))[0], INVALID),
    ("BIAS without bias", lambda L: plan(L, shape(), E["BIAS"])[0], INVALID),
    ("DEFAULT with stray bias", lambda L: plan(L, shape(), E["DEFAULT"], ep_epilog_io(bias=X_PTR))[0], INVALID),
    ("misaligned bias", lambda L: plan(L, shape(), E["RELU_BIAS"], ep_epilog_io(bias=X_PTR + 2))[0], INVALID),
    ("RELU_AUX_BIAS without relu_aux", lambda L: plan(L, shape(), E["RELU_AUX_BIAS"], ep_epilog_io(bias=X_PTR))[0], INVALID),
    ("ld_aux too small", lambda L: plan(L, shape(n=96, ldb=96, ldd=96), E["RELU_AUX_BIAS"],
                                        ep_epilog_io(bias=X_PTR, relu_aux=X_PTR + 4096, ld_aux=2))[0], INVALID),
    ("misaligned relu_aux", lambda L: plan(L, shape(), E["RELU_AUX_BIAS"],
                                           ep_epilog_io(bias=X_PTR, relu_aux=X_PTR + 4098))[0], INVALID),
    ("DRELU_BGRAD without bgrad", lambda L: plan(L, shape(lay=NK), E["DRELU_BGRAD"],
                                                 ep_epilog_io(relu_aux_in=X_PTR))[0], INVALID),
    ("DRELU_BGRAD without mask", lambda L: plan(L, shape(lay=NK), E["DRELU_BGRAD"],
                                                ep_epilog_io(bgrad=X_PTR))[0], INVALID),
    ("misaligned bgrad", lambda L: plan(L, shape(lay=NK), E["DRELU_BGRAD"],
                                        ep_epilog_io(relu_aux_in=X_PTR, bgrad=X_PTR + 4100))[0], INVALID),
    ("SWIGLU without b2", lambda L: plan(L, shape(lay=NK), E["SWIGLU"])[0], INVALID),
    ("DSWIGLU without up", lambda L: plan(L, shape(), E["DSWIGLU"], ep_epilog_io(gate=X_PTR, d2=X_PTR + 8192))[0], INVALID),
    ("DSWIGLU ld_gu too small", lambda L: plan(L, shape(), E["DSWIGLU"],
                                               ep_epilog_io(gate=X_PTR, up=X_PTR + 8192, d2=X_PTR + 16384, ld_gu=32))[0], INVALID),
    ("ld_gu on a non-DSWIGLU epilog", lambda L: plan(L, shape(), E["DEFAULT"], ep_epilog_io(ld_gu=64))[0], INVALID),
    ("unknown path", lambda L: plan(L, shape(), opt=ep_options(path=5, bgrad_mode=0, tile_cfg=-1))[0], INVALID),
    ("tile_cfg out of range", lambda L: plan(L, shape(), opt=ep_options(path=0, bgrad_mode=0, tile_cfg=99))[0], INVALID),
    ("unfused with atomic bgrad", lambda L: plan(L, shape(lay=NK), E["DRELU_BGRAD"],
                                                 ep_epilog_io(relu_aux_in=X_PTR, bgrad=X_PTR + 4096),
                                                 opt=ep_options(path=1, bgrad_mode=1, tile_cfg=-1))[0], UNSUPPORTED),
    ("split_k negative", lambda L: plan(L, shape(), opt=ep_options(path=0, bgrad_mode=0, tile_cfg=-1, split_k=-1))[0], INVALID),
    ("split_k above 8", lambda L: plan(L, shape(), opt=ep_options(path=0, bgrad_mode=0, tile_cfg=-1, split_k=9))[0], INVALID),
    ("split_tail not 0/1", lambda L: plan(L, shape(), opt=ep_options(path=0, bgrad_mode=0, tile_cfg=-1, split_k=2,
                                                                       split_tail=2))[0], INVALID),
    ("unfused with split_k", lambda L: plan(L, shape(), opt=ep_options(path=1, bgrad_mode=0, tile_cfg=-1, split_k=2))[0],
     UNSUPPORTED),
    ("unknown A layout", lambda L: plan(L, shape(alay=2))[0], UNSUPPORTED),
    ("K x M A with a non-DEFAULT epilog", lambda L: plan(L, shape(alay=1), E["BIAS"], ep_epilog_io(bias=X_PTR))[0],
     UNSUPPORTED),
    ("K x M A with m not a multiple of 8", lambda L: plan(L, shape(m=60, alay=1, lda=64))[0], UNSUPPORTED),
    ("K x M A with lda < m", lambda L: plan(L, shape(m=128, alay=1, lda=64))[0], INVALID),
    ("GELU_BIAS without bias", lambda L: plan(L, shape(), E["GELU_BIAS"])[0], INVALID),
    ("GELU_AUX_BIAS without gelu_aux", lambda L: plan(L, shape(), E["GELU_AUX_BIAS"], ep_epilog_io(bias=X_PTR))[0], INVALID),
    ("GELU_BIAS with a stray gelu_aux", lambda L: plan(L, shape(), E["GELU_BIAS"],
                                                       ep_epilog_io(bias=X_PTR, gelu_aux=X_PTR + 8192))[0], INVALID),
    ("misaligned gelu_aux", lambda L: plan(L, shape(), E["GELU_AUX_BIAS"],
                                           ep_epilog_io(bias=X_PTR, gelu_aux=X_PTR + 8200))[0], INVALID),
    ("ld_gelu_aux too small", lambda L: plan(L, shape(), E["GELU_AUX_BIAS"],
                                             ep_epilog_io(bias=X_PTR, gelu_aux=X_PTR + 8192, ld_gelu_aux=56))[0], INVALID),
    ("ld_gelu_aux not multiple of 8", lambda L: plan(L, shape(), E["GELU_AUX_BIAS"],
                                                     ep_epilog_io(bias=X_PTR, gelu_aux=X_PTR + 8192, ld_gelu_aux=68))[0], INVALID),
    ("DGELU_BGRAD without bgrad", lambda L: plan(L, shape(lay=NK), E["DGELU_BGRAD"], ep_epilog_io(gelu_aux=X_PTR))[0], INVALID),
    ("DGELU_BGRAD without gelu_aux", lambda L: plan(L, shape(lay=NK), E["DGELU_BGRAD"], ep_epilog_io(bgrad=X_PTR))[0], INVALID),
    ("ld_gelu_aux on a non-GELU epilog", lambda L: plan(L, shape(), E["DEFAULT"], ep_epilog_io(ld_gelu_aux=64))[0], INVALID),
    ("autotune not 0/1", lambda L: plan(L, shape(), opt=ep_options(path=0, bgrad_mode=0, tile_cfg=-1, autotune=2))[0], INVALID),
    ("autotune with a fixed tile_cfg", lambda L: plan(L, shape(), opt=ep_options(path=0, bgrad_mode=0, tile_cfg=0,
                                                                                   autotune=1))[0], INVALID),
    ("autotune with split_k", lambda L: plan(L, shape(), opt=ep_options(path=0, bgrad_mode=0, tile_cfg=-1, split_k=2,
                                                                          autotune=1))[0], INVALID),
    ("autotune on the unfused path", lambda L: plan(L, shape(), opt=ep_options(path=1, bgrad_mode=0, tile_cfg=-1,
                                                                                 autotune=1))[0], INVALID),
]


@pytest.mark.parametrize("name,call,want", CASES, ids=[c[0] for c in CASES])
def test_validation_rejects_before_hip(L, name, call, want):
    assert call(L) == want, f"{name}: {L.ep_last_error().decode()}"
    assert L.ep_last_error().decode() != ""


def test_null_out_pointer(L):
    s = shape()
    io = ep_epilog_io()
    assert L.ep_plan_ex(ctypes.byref(s), F16, 0, ctypes.byref(io), None, None) == INVALID


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


@pytest.mark.skipif(not _no_gpu(), reason="checks the no-device path")
def test_valid_plan_without_device_returns_hip_error(L):
    r, h = plan(L, shape(), E["DEFAULT"])
    assert r == HIP, L.ep_last_error().decode()
    assert h.value is None


def test_python_binding_rejects_bad_inputs():
    import torch
    a = torch.zeros((8, 8), dtype=torch.float32)
    with pytest.raises(ValueError):
        ep.Plan(a, a)
    h = torch.zeros((8, 8), dtype=torch.float16)
    with pytest.raises(ValueError):
        ep.Plan(h, h, epilog="NOT_AN_EPILOG")
