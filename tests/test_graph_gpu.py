"""ep_execute captured in a HIP graph: every replay must reproduce the eager result exactly.

The fused kernels are deterministic (two-pass bias gradient, split-K partials summed in a
fixed order), so a replay is compared bit for bit with an eager execution on the same
inputs.  Each replay is preceded by unrelated eager work, a synchronisation and an
overwrite of the outputs, so a replay that skipped or reordered a node would show.
"""
import pytest
import torch

from tests._gpu import require_gpu, say

pytestmark = pytest.mark.gpu


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _check_replays(g, outs, refs, what):
    junk = torch.empty(1 << 20, device="cuda")
    for r in range(3):
        junk.normal_()                       # unrelated eager work between replays
        torch.cuda.synchronize()
        for o in outs:
            o.view(torch.uint8).fill_(0xA5)  # outputs must be rewritten by the replay
        g.replay()
        torch.cuda.synchronize()
        for o, ref, name in zip(outs, refs, what):
            assert torch.equal(o.view(torch.uint8), ref.view(torch.uint8)), f"replay {r}: {name} differs"


def _rand(shape, dt, seed, scale=1.0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.randn(shape, device="cuda", generator=g) * scale).to(dt)


def test_graph_relu_layer_forward_backward():
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    say("case graph: RELU_AUX_BIAS forward + DRELU_BGRAD backward, fp16 1024x768x512")
    m, n, k = 1024, 768, 512
    x, w, bias = _rand((m, k), torch.float16, 1), _rand((k, n), torch.float16, 2, 0.05), _rand((n,), torch.float16, 3, 0.1)
    dy = _rand((m, n), torch.float16, 4)
    pf = ep.Plan(x, w, "RELU_AUX_BIAS", {"bias": bias}, b_layout="KN")
    y, aux = pf.execute()
    # backward dX = mask * (dY . W^T): W (k x n) is the N x K operand; a separate mask of
    # m x k bits stands for the previous layer's relu_aux
    g0 = torch.Generator(device="cuda")
    g0.manual_seed(10)
    mask = torch.randint(-2**31, 2**31, (m, k // 32), device="cuda", dtype=torch.int64, generator=g0).to(torch.int32)
    pb = ep.Plan(dy, w, "DRELU_BGRAD", {"relu_aux": mask}, b_layout="NK")
    dx, auxb = pb.execute()
    torch.cuda.synchronize()
    refs = [y.clone(), aux["relu_aux"].clone(), dx.clone(), auxb["drelu_bgrad"].clone()]
    g = _capture(lambda: (pf.execute(), pb.execute()))
    _check_replays(g, [y, aux["relu_aux"], dx, auxb["drelu_bgrad"]], refs, ["Y", "relu_aux", "dX", "bgrad"])
    pf.free()
    pb.free()


def test_graph_split_k_and_swiglu():
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    say("case graph: split-K DEFAULT bf16 512x1024x8192 (3 splits) and SWIGLU bf16 512x1024x640")
    a, b = _rand((512, 8192), torch.bfloat16, 5), _rand((1024, 8192), torch.bfloat16, 6, 0.02)
    p1 = ep.Plan(a, b, "DEFAULT", b_layout="NK", split_k=3)
    assert "splits=3 " in p1.info()
    d1, _ = p1.execute()
    x, wg, wu = _rand((512, 640), torch.bfloat16, 7), _rand((1024, 640), torch.bfloat16, 8, 0.05), _rand((1024, 640), torch.bfloat16, 9, 0.05)
    p2 = ep.Plan(x, wg, "SWIGLU", {"b2": wu}, b_layout="NK")
    h, _ = p2.execute()
    torch.cuda.synchronize()
    refs = [d1.clone(), h.clone()]
    g = _capture(lambda: (p1.execute(), p2.execute()))
    _check_replays(g, [d1, h], refs, ["split-K D", "SwiGLU h"])
    p1.free()
    p2.free()
