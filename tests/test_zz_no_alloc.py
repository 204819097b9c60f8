"""ep_execute_noalloc, the entry point for callers that cannot allocate, against the plan/execute
entry points on the same inputs.

It plans exactly as ep_plan_ex does and runs the same kernels, with its workspace (two-pass
bias-gradient partials, split-K partial tiles) in a static device array instead of a plan-owned
allocation, so its outputs must equal ep_execute's bit for bit, and the oracle's within the
usual tolerances.  Each case runs twice in a row, the second time on a smaller problem, so that
stale scratch contents from the first call would show.  Calls go through the C ABI (ctypes).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from tests._gpu import assert_bgrad, assert_half, assert_mask, f64, require_gpu, say, words

pytestmark = pytest.mark.gpu

F16, BF16 = 0, 1


def _ep():
    import dense_gemm_epilogues_amd as ep
    return ep


def noalloc(L, shape, dtype, epi, io, opt, stream=None):
    L.ep_execute_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    L.ep_execute_noalloc.restype = ctypes.c_int
    s = torch.cuda.current_stream() if stream is None else stream
    return L.ep_execute_noalloc(ctypes.byref(shape), dtype, epi, ctypes.byref(io),
                                ctypes.byref(opt) if opt is not None else None, ctypes.c_void_p(s.cuda_stream))


def ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def drelu_case(m, n, k, seed, split_k=0, expect_split=False):
    """DRELU_BGRAD two-pass (and optionally split-K): dX and bgrad from both entry points."""
    ep = _ep()
    L = ep.lib()
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(seed)
    dy = torch.randn(m, k, generator=g).half().to(dev)              # A: m x k
    w = (torch.randn(n, k, generator=g) * k ** -0.5).half().to(dev)  # B given N x K
    mask = torch.from_numpy(oracle.pack_relu_mask(torch.randn(m, n, generator=g).numpy() > 0).view(np.int32).copy()).to(dev)
    ref_plan = ep.Plan(dy, w, "DRELU_BGRAD", {"relu_aux": mask}, b_layout="NK", split_k=split_k)
    if expect_split:
        assert int(ref_plan.info().split("splits=")[1].split()[0]) > 1, ref_plan.info()
    dx_ref, aux = ref_plan.execute()
    bg_ref = aux["drelu_bgrad"]
    dx = torch.full((m, n), float("nan"), dtype=torch.float16, device=dev)
    bg = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    shape = ep.ep_shape(m=m, n=n, k=k, b_layout=1, a=ptr(dy), lda=k, b=ptr(w), ldb=k, d=ptr(dx), ldd=n, a_layout=0)
    io = ep.ep_epilog_io(relu_aux_in=ptr(mask), ld_aux=mask.stride(0), bgrad=ptr(bg))
    opt = ep.ep_options(path=0, bgrad_mode=0, tile_cfg=-1, split_k=split_k, autotune=0)
    st = noalloc(L, shape, F16, ep.EPILOGS["DRELU_BGRAD"], io, opt)
    assert st == 0, L.ep_last_error().decode()
    torch.cuda.synchronize()
    what = f"noalloc DRELU_BGRAD {m}x{n}x{k} split {split_k} ({ref_plan.info()})"
    assert torch.equal(dx.view(torch.int16), dx_ref.view(torch.int16)), what + ": dX differs from ep_execute"
    assert torch.equal(bg.view(torch.int32), bg_ref.view(torch.int32)), what + ": bgrad differs from ep_execute"
    dxo, bgo = oracle.drelu_bgrad(f64(dy), f64(w), "NK", words(mask))
    assert_half(f64(dx), dxo, what)
    assert_bgrad(bg.cpu().numpy(), bgo, what)
    ref_plan.free()


def relu_aux_case(m, n, k, seed, split_k, split_tail=False, tile_cfg=-1):
    ep = _ep()
    L = ep.lib()
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(m, k, generator=g).to(torch.bfloat16).to(dev)
    w = (torch.randn(k, n, generator=g) * k ** -0.5).to(torch.bfloat16).to(dev)
    bias = (torch.randn(n, generator=g) * 0.1).to(torch.bfloat16).to(dev)
    ref_plan = ep.Plan(x, w, "RELU_AUX_BIAS", {"bias": bias}, b_layout="KN", split_k=split_k, split_tail=split_tail,
                       tile_cfg=tile_cfg)
    if split_tail:
        assert "split_tail0=256 " in ref_plan.info(), ref_plan.info()
    y_ref, aux = ref_plan.execute()
    nw = (n + 31) // 32
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=dev)
    words_out = torch.full((m, nw), -1, dtype=torch.int32, device=dev)
    shape = ep.ep_shape(m=m, n=n, k=k, b_layout=0, a=ptr(x), lda=k, b=ptr(w), ldb=n, d=ptr(y), ldd=n, a_layout=0)
    io = ep.ep_epilog_io(bias=ptr(bias), relu_aux=ptr(words_out), ld_aux=nw)
    opt = ep.ep_options(path=0, bgrad_mode=0, tile_cfg=tile_cfg, split_k=split_k, split_tail=int(split_tail), autotune=0)
    st = noalloc(L, shape, BF16, ep.EPILOGS["RELU_AUX_BIAS"], io, opt)
    assert st == 0, L.ep_last_error().decode()
    torch.cuda.synchronize()
    what = f"noalloc RELU_AUX_BIAS {m}x{n}x{k} split {split_k} ({ref_plan.info()})"
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), what + ": Y differs from ep_execute"
    assert torch.equal(words_out, aux["relu_aux"]), what + ": mask words differ from ep_execute"
    yo, _, pre = oracle.relu_aux_bias(f64(x), f64(w), f64(bias), "KN")
    assert_half(f64(y), yo, what)
    assert_mask(words(words_out), pre, what)
    ref_plan.free()


def test_noalloc_drelu_bgrad_two_calls():
    """Two-pass bias-gradient partials in the static scratch: the square layer's size, then a
    smaller ragged problem on the same scratch."""
    require_gpu()
    say("case noalloc DRELU_BGRAD 4096^3 then 300x200x136")
    drelu_case(4096, 4096, 4096, seed=1)
    drelu_case(300, 200, 136, seed=2)


def test_noalloc_split_k_two_calls():
    """Split-K partial tiles in the static scratch (forced 3 and chosen by shape), then smaller."""
    require_gpu()
    say("case noalloc split-K RELU_AUX_BIAS and DRELU_BGRAD")
    relu_aux_case(1024, 1024, 8192, seed=3, split_k=3)
    relu_aux_case(260, 296, 520, seed=4, split_k=2)
    drelu_case(1024, 768, 34816, seed=5, split_k=0, expect_split=True)  # few long-K tiles: split by shape
    drelu_case(130, 264, 520, seed=6, split_k=2)


def test_noalloc_split_tail_two_calls():
    """A split of the last round's tiles only (272 256x256 tiles of configuration 11: 256 whole,
    16 split 3 ways), its partials in the static scratch, then a smaller uniformly split
    problem."""
    require_gpu()
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the tail's position assumes 256 CUs")
    say("case noalloc split tail RELU_AUX_BIAS 4312x4072x512, then 260x296x520")
    relu_aux_case(4312, 4072, 512, seed=7, split_k=3, split_tail=True, tile_cfg=11)
    relu_aux_case(260, 296, 520, seed=8, split_k=2)


def test_noalloc_rejects_oversized_workspace_and_unsupported_options():
    """A forced split whose partials exceed the scratch, the unfused path and autotune are
    refused before anything is launched (outputs untouched)."""
    require_gpu()
    ep = _ep()
    L = ep.lib()
    dev = torch.device("cuda")
    m, n, k = 256 * 13, 256 * 5, 4 * 32                  # 65 output tiles
    assert 4 * 65 * 256 * 256 * 4 > (64 << 20)          # 4 splits of partial tiles: 65 MiB
    x = torch.zeros(m, k, dtype=torch.float16, device=dev)
    w = torch.zeros(k, n, dtype=torch.float16, device=dev)
    y = torch.full((m, n), 7.0, dtype=torch.float16, device=dev)
    shape = ep.ep_shape(m=m, n=n, k=k, b_layout=0, a=ptr(x), lda=k, b=ptr(w), ldb=n, d=ptr(y), ldd=n, a_layout=0)
    io = ep.ep_epilog_io()
    say("case noalloc refusals")
    st = noalloc(L, shape, F16, 0, io, ep.ep_options(path=0, bgrad_mode=0, tile_cfg=0, split_k=4, autotune=0))
    assert st == 2 and "workspace" in L.ep_last_error().decode(), (st, L.ep_last_error())
    st = noalloc(L, shape, F16, 0, io, ep.ep_options(path=1, bgrad_mode=0, tile_cfg=-1, split_k=0, autotune=0))
    assert st == 2 and "unfused" in L.ep_last_error().decode()
    st = noalloc(L, shape, F16, 0, io, ep.ep_options(path=0, bgrad_mode=0, tile_cfg=-1, split_k=0, autotune=1))
    assert st == 1 and "autotune" in L.ep_last_error().decode()
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a refused call wrote its output"
    # the same problem unsplit fits and runs
    st = noalloc(L, shape, F16, 0, io, ep.ep_options(path=0, bgrad_mode=0, tile_cfg=0, split_k=1, autotune=0))
    assert st == 0, L.ep_last_error().decode()
    torch.cuda.synchronize()
    assert int((y.view(torch.int16) != 0).sum()) == 0
