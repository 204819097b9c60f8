"""Fusion evidence and memory behaviour on the GPU.

Launch counts: the cudnn-frontend SwiGLU sample (gemm_swiglu_mlp_fusion.py, _demo) counts
the GPU launches of one fused call with a profiler, so that "one kernel" is observed, not
assumed.  Here torch.profiler records the kernels that one ep_execute enqueues:
RELU_AUX_BIAS, SWIGLU and DSWIGLU are one kernel each; DRELU_BGRAD is the GEMM plus the
bias-gradient pass (two-pass) or a zero fill plus the GEMM (atomic); split-K adds the
fixup launch; the unfused baseline runs its separate kernels, e.g. GEMM, bias add and ReLU
for the forward ("three independent kernels" in the hotdry.top post, paragraph 8).

Memory behaviour ("Suitable evaluation scenarios" of Fusing Matmul Epilogs with
nvmath-python lists validating memory behaviour): repeated executes and plan/free cycles
leave the device's free memory unchanged, and the deterministic two-pass bias gradient is
bitwise repeatable.
"""
import numpy as np
import pytest
import torch
from torch.profiler import ProfilerActivity, profile

import workloads as W
from tests._gpu import require_gpu, say

pytestmark = pytest.mark.gpu


def _ep():
    import dense_gemm_epilogues_amd as ep
    return ep


def kernels_of(fn):
    """Names of the GPU kernels that fn() enqueues (after one warm call outside the trace)."""
    fn()
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    names = []
    for e in prof.events():
        if e.device_type == torch.autograd.DeviceType.CUDA and "Memcpy" not in e.name and "Memset" not in e.name:
            names.append(e.name)
    return names


def inputs(dt, m=512, n=384, k=256, dev="cuda"):
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    r = lambda *s, sc=1.0: (torch.randn(*s, device=dev, generator=g) * sc).to(dt)
    return {"x": r(m, k), "w_kn": r(k, n, sc=k ** -0.5), "w_nk": r(n, k, sc=k ** -0.5),
            "w2_nk": r(n, k, sc=k ** -0.5), "bias": r(n, sc=0.1), "gate": r(m, n), "up": r(m, n),
            "mask": torch.randint(-2 ** 31, 2 ** 31 - 1, (m, (n + 31) // 32), device=dev, dtype=torch.int32,
                                  generator=g)}


CASES = [
    # (name, epilog, layout, options, expected kernel names in order (substrings))
    ("RELU_AUX_BIAS", "RELU_AUX_BIAS", "KN", {}, ["gemm_kernel"]),
    ("SWIGLU", "SWIGLU", "NK", {}, ["gemm_kernel"]),
    ("DSWIGLU", "DSWIGLU", "KN", {}, ["gemm_kernel"]),
    ("DRELU_BGRAD two-pass", "DRELU_BGRAD", "NK", {}, ["gemm_kernel", "bgrad_reduce"]),
    ("DRELU_BGRAD atomic", "DRELU_BGRAD", "NK", {"bgrad_mode": "atomic"}, ["fill_zero", "gemm_kernel"]),
    ("RELU_AUX_BIAS split-K", "RELU_AUX_BIAS", "KN", {"split_k": 2}, ["gemm_kernel", "gemm_kernel"]),
    ("DRELU_BGRAD split-K", "DRELU_BGRAD", "NK", {"split_k": 2}, ["gemm_kernel", "gemm_kernel", "bgrad_reduce"]),
    ("unfused RELU_AUX_BIAS", "RELU_AUX_BIAS", "KN", {"path": "unfused"}, ["gemm_kernel", "bias_add", "relu_pack"]),
    ("unfused DRELU_BGRAD", "DRELU_BGRAD", "NK", {"path": "unfused"},
     ["gemm_kernel", "mask_apply", "colsum", "bgrad_reduce"]),
    ("unfused SWIGLU", "SWIGLU", "NK", {"path": "unfused"}, ["gemm_kernel", "gemm_kernel", "silu_mul"]),
    ("unfused DSWIGLU", "DSWIGLU", "KN", {"path": "unfused"}, ["gemm_kernel", "dswiglu"]),
]


@pytest.mark.parametrize("name,epi,layout,opts,want", CASES, ids=[c[0] for c in CASES])
def test_launch_count(name, epi, layout, opts, want):
    require_gpu()
    ep = _ep()
    dt = torch.bfloat16 if "SWIGLU" in epi else torch.float16
    ins = inputs(dt)
    b = ins["w_kn"] if layout == "KN" else ins["w_nk"]
    epi_in = {"BIAS": {"bias": ins["bias"]}, "RELU_AUX_BIAS": {"bias": ins["bias"]},
              "DRELU_BGRAD": {"relu_aux": ins["mask"]}, "SWIGLU": {"b2": ins["w2_nk"]},
              "DSWIGLU": {"gate": ins["gate"], "up": ins["up"]}}[epi]
    say(f"case launch count {name}")
    p = ep.Plan(ins["x"], b, epi, epi_in, b_layout=layout, **opts)
    names = kernels_of(p.execute)
    p.free()
    assert len(names) == len(want), f"{name}: {len(names)} kernels {names}, expected {want}"
    for got, w in zip(names, want):
        assert w in got, f"{name}: kernel {got!r} where {w!r} was expected ({names})"


def test_bgrad_two_pass_bitwise_repeatable():
    """Ten eager executes of the square layer's DRELU_BGRAD (two-pass bias gradient) give
    bitwise identical dX and bgrad; so do ten executes of the forward."""
    require_gpu()
    ep = _ep()
    dev = torch.device("cuda")
    c = W.LINEAR[2]
    inp = W.linear_inputs(c, device=dev)
    pf = ep.Plan(inp["x"], inp["w"], "RELU_AUX_BIAS", {"bias": inp["bias"]}, b_layout="KN")
    y0, aux0 = pf.execute()
    y0, m0 = y0.clone(), aux0["relu_aux"].clone()
    pb = ep.Plan(inp["dy"], inp["w"], "DRELU_BGRAD", {"relu_aux": m0}, b_layout="NK")
    dx0, auxb = pb.execute()
    dx0, bg0 = dx0.clone(), auxb["drelu_bgrad"].clone()
    for i in range(10):
        say(f"case repeatability run {i}")
        y, aux = pf.execute()
        dx, auxb = pb.execute()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), f"run {i}: forward Y differs"
        assert torch.equal(aux["relu_aux"], m0), f"run {i}: relu_aux differs"
        assert torch.equal(dx.view(torch.int16), dx0.view(torch.int16)), f"run {i}: dX differs"
        assert torch.equal(auxb["drelu_bgrad"].view(torch.int32), bg0.view(torch.int32)), f"run {i}: bgrad differs"
    pf.free()
    pb.free()


def test_no_device_memory_growth():
    """1000 executes and 100 plan/free cycles (every workspace kind: two-pass bias-gradient
    partials, split-K partials, the unfused path's intermediates) leave the device's free
    memory (hipMemGetInfo) unchanged.  Outputs are preallocated, so the only allocations in
    the loop are the library's own."""
    require_gpu()
    ep = _ep()
    dev = torch.device("cuda")
    f16, bf16 = inputs(torch.float16), inputs(torch.bfloat16)
    m, n = f16["x"].shape[0], f16["w_kn"].shape[1]
    outs = {"y": torch.empty(m, n, dtype=torch.float16, device=dev),
            "yb": torch.empty(m, n, dtype=torch.bfloat16, device=dev),
            "bg": torch.empty(n, dtype=torch.float32, device=dev),
            "mask": torch.empty(m, (n + 31) // 32, dtype=torch.int32, device=dev)}
    specs = [
        (f16["x"], f16["w_nk"], "DRELU_BGRAD", {"relu_aux": f16["mask"]}, "NK", {}, outs["y"], {"drelu_bgrad": outs["bg"]}),
        (f16["x"], f16["w_kn"], "RELU_AUX_BIAS", {"bias": f16["bias"]}, "KN", {"split_k": 3}, outs["y"],
         {"relu_aux": outs["mask"]}),
        (f16["x"], f16["w_nk"], "DRELU_BGRAD", {"relu_aux": f16["mask"]}, "NK", {"path": "unfused"}, outs["y"],
         {"drelu_bgrad": outs["bg"]}),
        (bf16["x"], bf16["w_nk"], "SWIGLU", {"b2": bf16["w2_nk"]}, "NK", {"path": "unfused"}, outs["yb"], {}),
    ]

    def cycle():
        for (a, b, epi, ins, lay, opts, out, aux) in specs:
            p = ep.Plan(a, b, epi, ins, b_layout=lay, out=out, aux_out=aux, **opts)
            p.execute()
            p.free()

    cycle()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    say(f"case memory: free before {free0}")
    for i in range(100):
        cycle()
    torch.cuda.synchronize()
    (a, b, epi, ins, lay, opts, out, aux) = specs[0]
    p = ep.Plan(a, b, epi, ins, b_layout=lay, out=out, aux_out=aux, **opts)
    for i in range(1000):
        p.execute()
    torch.cuda.synchronize()
    p.free()
    free1, _ = torch.cuda.mem_get_info()
    say(f"case memory: free after {free1}")
    assert free1 == free0, f"device free memory changed by {free1 - free0} bytes"
