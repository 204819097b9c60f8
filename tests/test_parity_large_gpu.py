"""GPU parity at the full sizes of the four large workloads, in the launch configuration the
benchmark times (default plan, tile configuration chosen by the library).

  * square fp16 layer 4096^3: forward and backward compared in full with the oracle;
  * H200-shape fp16 layer (65536 x 16384 x 8192): seeded 128x128 output tiles and bias-
    gradient columns against the oracle, all 16384 bgrad columns against the all-ones-mask
    closed form, the all-zeros mask exactly, and the ReLU/mask invariants on every element;
  * bf16 SwiGLU forward (M 2048, H 5120, I 17408): h and the down projection in full;
  * bf16 GEMM + dSwiGLU backward (M 16384): seeded tiles of d_gate and d_up.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests._gpu import assert_bgrad, assert_half, assert_mask, f64, require_gpu, say, words

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _ep():
    import dense_gemm_epilogues_amd as ep
    return ep


def mask_bits_gpu(wd, n):
    """(M, ceil(n/32)) int32 words -> (M, n) uint8 bits, on the device."""
    sh = torch.arange(32, device=wd.device, dtype=torch.int32)
    bits = (wd.unsqueeze(-1) >> sh) & 1
    return bits.reshape(wd.shape[0], -1)[:, :n].to(torch.uint8)


def relu_invariants_gpu(y, wd, n, what):
    bits = mask_bits_gpu(wd, n)
    yb = y.view(torch.int16)
    assert int(((bits == 0) & (yb != 0)).sum()) == 0, f"{what}: masked-out element not +0"
    assert int((y.float() < 0).sum()) == 0, f"{what}: negative output after ReLU"
    assert int((yb == -32768).sum()) == 0, f"{what}: -0 emitted"
    tail = n % 32
    if tail:
        assert int((wd[:, -1] >> tail).sum()) == 0, f"{what}: tail bits set"


# ------------------------------------------------------------------ square 4096 layer
def test_square_layer_full():
    require_gpu()
    ep = _ep()
    c = W.LINEAR[2]
    dev = torch.device("cuda")
    say("case square layer 4096^3 fp16: forward RELU_AUX_BIAS")
    inp = W.linear_inputs(c, device=dev)
    x, w, bias, dy = inp["x"], inp["w"], inp["bias"], inp["dy"]
    pf = ep.Plan(x, w, "RELU_AUX_BIAS", {"bias": bias}, b_layout="KN")
    y, aux = pf.execute()
    torch.cuda.synchronize()
    x64, w64, b64, dy64 = f64(x), f64(w), f64(bias), f64(dy)
    yref, wref, pre = oracle.relu_aux_bias(x64, w64, b64, "KN")
    assert_half(f64(y), yref, "square fwd Y")
    assert_mask(words(aux["relu_aux"]), pre, "square fwd relu_aux")
    relu_invariants_gpu(y, aux["relu_aux"], c.n, "square fwd")

    # backward consumes the oracle's own mask (an input both sides share)
    say("case square layer 4096^3 fp16: backward DRELU_BGRAD")
    mask_in = torch.from_numpy(wref.view(np.int32).copy()).to(dev)
    pb = ep.Plan(dy, w, "DRELU_BGRAD", {"relu_aux": mask_in}, b_layout="NK")
    dx, auxb = pb.execute()
    torch.cuda.synchronize()
    dxref, bgref = oracle.drelu_bgrad(dy64, w64, "NK", wref)
    assert_half(f64(dx), dxref, "square bwd dX")
    assert_bgrad(auxb["drelu_bgrad"].cpu().numpy(), bgref, "square bwd bgrad")

    # chained: the backward fed with the GPU forward's mask differs from the one fed with
    # the oracle's mask only in columns of elements in the mask tolerance band
    pc = ep.Plan(dy, w, "DRELU_BGRAD", {"relu_aux": aux["relu_aux"]}, b_layout="NK")
    dx2, _ = pc.execute()
    torch.cuda.synchronize()
    differ = words(aux["relu_aux"]) != wref
    rows_changed = np.flatnonzero(differ.any(axis=1))
    same_rows = np.setdiff1d(np.arange(c.m), rows_changed)
    assert torch.equal(dx2[torch.from_numpy(same_rows).to(dev)], dx[torch.from_numpy(same_rows).to(dev)])
    for p in (pf, pb, pc):
        p.free()


# ------------------------------------------------------------------ H200-shape layer
def _h200_inputs(dev):
    c = W.LINEAR[3]
    return c, W.linear_inputs(c, device=dev)


def test_h200_layer_forward_sampled():
    require_gpu()
    ep = _ep()
    dev = torch.device("cuda")
    say("case H200 layer fp16 65536x16384x8192: forward RELU_AUX_BIAS")
    c, inp = _h200_inputs(dev)
    x, w, bias = inp["x"], inp["w"], inp["bias"]
    p = ep.Plan(x, w, "RELU_AUX_BIAS", {"bias": bias}, b_layout="KN")
    y, aux = p.execute()
    torch.cuda.synchronize()
    relu_invariants_gpu(y, aux["relu_aux"], c.n, "h200 fwd")
    b64 = f64(bias)
    for (r0, r1, c0, c1) in oracle.sample_tiles(c.m, c.n, count=32, seed=31):
        a64 = f64(x[r0:r1])
        w64 = f64(w[:, c0:c1])
        yref, _, pre = oracle.relu_aux_bias(a64, w64, b64[c0:c1], "KN")
        what = f"h200 fwd tile {(r0, c0)}"
        assert_half(f64(y[r0:r1, c0:c1]), yref, what)
        wsl = words(aux["relu_aux"][r0:r1, c0 // 32:(c1 + 31) // 32])
        assert_mask(wsl, pre, what)
    p.free()


def test_h200_layer_backward_sampled_and_closed_forms():
    require_gpu()
    ep = _ep()
    dev = torch.device("cuda")
    say("case H200 layer fp16: backward DRELU_BGRAD (separate relu_aux, sampled)")
    c, inp = _h200_inputs(dev)
    dy, w, mask_in = inp["dy"], inp["w"], inp["mask_in"]
    m, n_out, n_in = c.m, c.n, c.k  # dY is m x n_out, dX is m x n_in
    p = ep.Plan(dy, w, "DRELU_BGRAD", {"relu_aux": mask_in}, b_layout="NK")
    dx, aux = p.execute()
    torch.cuda.synchronize()
    bg = aux["drelu_bgrad"].cpu().numpy().astype(np.float64)
    w64_all = f64(w)  # n_in x n_out
    words_all = words(mask_in)
    for (r0, r1, c0, c1) in oracle.sample_tiles(m, n_in, count=32, seed=37):
        # tile columns start on a mask-word boundary (sample_tiles aligns them to 32)
        dxref, _ = oracle.drelu_bgrad(f64(dy[r0:r1]), w64_all[c0:c1], "NK",
                                      words_all[r0:r1, c0 // 32:(c1 + 31) // 32])
        assert_half(f64(dx[r0:r1, c0:c1]), dxref, f"h200 bwd tile {(r0, c0)}")
    # sampled bgrad columns: full column sums of the masked product, rows in chunks
    cols = oracle.sample_columns(n_in, count=64, seed=41)
    ref = np.zeros(len(cols))
    for r0 in range(0, m, 8192):
        g = oracle.matmul(f64(dy[r0:r0 + 8192]), w64_all[cols], "NK")
        bits = oracle.unpack_relu_mask(words_all[r0:r0 + 8192], n_in)[:, cols]
        ref += np.where(bits, g, 0.0).sum(axis=0)
    assert_bgrad(bg[cols], ref, "h200 bwd sampled bgrad")

    # all-ones mask: every bgrad column against the closed form colsum(dY) W^T
    say("case H200 layer fp16: backward with all-ones and all-zeros masks")
    ones = torch.full_like(mask_in, -1)
    p1 = ep.Plan(dy, w, "DRELU_BGRAD", {"relu_aux": ones}, b_layout="NK")
    _, aux1 = p1.execute()
    torch.cuda.synchronize()
    colsum = np.zeros(n_out)
    for r0 in range(0, m, 8192):
        colsum += f64(dy[r0:r0 + 8192]).sum(axis=0)
    cf = w64_all @ colsum
    assert_bgrad(aux1["drelu_bgrad"].cpu().numpy(), cf, "h200 bwd all-ones closed form")
    zeros = torch.zeros_like(mask_in)
    p0 = ep.Plan(dy, w, "DRELU_BGRAD", {"relu_aux": zeros}, b_layout="NK")
    dx0, aux0 = p0.execute()
    torch.cuda.synchronize()
    assert int((dx0.view(torch.int16) != 0).sum()) == 0, "all-zeros mask: dX not +0"
    assert int((aux0["drelu_bgrad"] != 0).sum()) == 0, "all-zeros mask: bgrad not 0"
    for q in (p, p1, p0):
        q.free()


# ------------------------------------------------------------------ SwiGLU forward
def test_swiglu_forward_full():
    require_gpu()
    ep = _ep()
    dev = torch.device("cuda")
    c = W.SWIGLU[4]
    say("case SwiGLU forward bf16 M2048 H5120 I17408")
    inp = W.swiglu_inputs(c, device=dev)
    x, wg, wu, wd = inp["x"], inp["wg"], inp["wu"], inp["wd"]
    ps = ep.Plan(x, wg, "SWIGLU", {"b2": wu}, b_layout="NK")
    h, _ = ps.execute()
    pd = ep.Plan(h, wd, "DEFAULT", b_layout="NK")
    out, _ = pd.execute()
    torch.cuda.synchronize()
    href, _, _ = oracle.swiglu(f64(x), f64(wg), f64(wu))
    assert_half(f64(h), href, "swiglu h")
    h_gpu = f64(h)
    assert_half(f64(out), oracle.matmul(h_gpu, f64(wd), "NK"), "down projection on the GPU's h")
    ps.free()
    pd.free()


# ------------------------------------------------------------------ dSwiGLU backward
def test_dswiglu_backward_sampled():
    require_gpu()
    ep = _ep()
    dev = torch.device("cuda")
    c = W.SWIGLU[5]
    say("case GEMM + dSwiGLU backward bf16 M16384 H5120 I17408")
    inp = W.dswiglu_inputs(c, device=dev)
    dout, wd, gate, up = inp["dout"], inp["wd"], inp["gate"], inp["up"]
    p = ep.Plan(dout, wd, "DSWIGLU", {"gate": gate, "up": up}, b_layout="KN")
    dg, aux = p.execute()
    torch.cuda.synchronize()
    du = aux["d_up"]
    for (r0, r1, c0, c1) in oracle.sample_tiles(c.m, c.i, count=32, seed=53):
        dgr, dur, _ = oracle.dswiglu(f64(dout[r0:r1]), f64(wd[:, c0:c1]), f64(gate[r0:r1, c0:c1]),
                                     f64(up[r0:r1, c0:c1]))
        assert_half(f64(dg[r0:r1, c0:c1]), dgr, f"dswiglu d_gate tile {(r0, c0)}")
        assert_half(f64(du[r0:r1, c0:c1]), dur, f"dswiglu d_up tile {(r0, c0)}")
    assert bool(torch.isfinite(dg.float()).all()) and bool(torch.isfinite(du.float()).all())
    p.free()


# ------------------------------------------------------------------ GELU layer (square 4096)
def test_square_gelu_layer_full():
    """GELU_AUX_BIAS forward and DGELU_BGRAD backward on the square fp16 layer's inputs,
    compared in full; the backward consumes the pre-activation the GPU forward saved."""
    require_gpu()
    ep = _ep()
    c = W.LINEAR[2]
    dev = torch.device("cuda")
    say("case square GELU layer 4096^3 fp16: forward GELU_AUX_BIAS, backward DGELU_BGRAD")
    inp = W.linear_inputs(c, device=dev)
    x, w, bias, dy = inp["x"], inp["w"], inp["bias"], inp["dy"]
    pf = ep.Plan(x, w, "GELU_AUX_BIAS", {"bias": bias}, b_layout="KN")
    y, aux = pf.execute()
    pb = ep.Plan(dy, w, "DGELU_BGRAD", {"gelu_aux": aux["gelu_aux"]}, b_layout="NK")
    dx, auxb = pb.execute()
    torch.cuda.synchronize()
    x64, w64, b64, dy64 = f64(x), f64(w), f64(bias), f64(dy)
    yref, pref = oracle.gelu_aux_bias(x64, w64, b64, "KN")
    assert_half(f64(y), yref, "square gelu fwd Y")
    assert_half(f64(aux["gelu_aux"]), pref, "square gelu fwd pre-activation")
    dxref, bgref = oracle.dgelu_bgrad(dy64, w64, "NK", f64(aux["gelu_aux"]))
    assert_half(f64(dx), dxref, "square gelu bwd dX")
    assert_bgrad(auxb["dgelu_bgrad"].cpu().numpy(), bgref, "square gelu bwd bgrad")
    # a zero pre-activation: gelu'(0) = 1/2, so bgrad is half the all-ones closed form
    zeros = torch.zeros_like(aux["gelu_aux"])
    p0 = ep.Plan(dy, w, "DGELU_BGRAD", {"gelu_aux": zeros}, b_layout="NK")
    _, aux0 = p0.execute()
    torch.cuda.synchronize()
    cf = 0.5 * oracle.bgrad_all_ones_closed_form(dy64, w64, "NK")
    assert_bgrad(aux0["dgelu_bgrad"].cpu().numpy(), cf, "square gelu bwd, zero pre-activation closed form")
    for p in (pf, pb, p0):
        p.free()


# ------------------------------------------------------------------ SwiGLU-MLP training step
def test_swiglu_mlp_training_step_all_gradients():
    """The whole SwiGLU MLP forward and backward with this library only, M 2048:
      forward  h and the saved [g | u] = SWIGLU_AUX(x; Wg, Wu) (W_gu = [Wg; Wu]), out = h Wd^T, and
               the recompute alternative [g | u] = x W_gu^T (one DEFAULT GEMM) as a cross-check;
      backward [d_gate | d_up] = DSWIGLU(dout, Wd; g, u) into one M x 2I buffer,
               dx = [d_gate | d_up] . W_gu  (one GEMM over the concatenated K = 2I),
               [dWg; dWu] = [d_gate | d_up]^T . x and dWd = dout^T . h (transposed-A GEMMs).
    Every step is compared with the oracle applied to the same inputs the GPU step consumed
    (the previous GPU step's output), so each kernel is checked on its own, on sampled tiles
    that cover every region of its output."""
    require_gpu()
    ep = _ep()
    dev = torch.device("cuda")
    c = W.SWIGLU[4]
    m, hd, idim = c.m, c.h, c.i
    say("case SwiGLU-MLP training step bf16 M2048 H5120 I17408: all four gradients")
    inp = W.swiglu_inputs(c, device=dev)
    x, wg, wu, wd = inp["x"], inp["wg"], inp["wu"], inp["wd"]
    w_gu = torch.cat([wg, wu], dim=0).contiguous()                     # 2I x H
    dout = W.randn((m, hd), W.seed_of(c.cfg, 6), 1.0, torch.bfloat16, dev)
    plans = []

    def run(*args, **kw):
        p = ep.Plan(*args, **kw)
        plans.append(p)  # kept until the device is synchronised
        return p.execute()[0]

    # forward (saving): h and [g | u] from one kernel
    ps = ep.Plan(x, w_gu[:idim], "SWIGLU_AUX", {"b2": w_gu[idim:]}, b_layout="NK")
    plans.append(ps)
    h, aux = ps.execute()
    gu = aux["gu"]                                                       # M x 2I = [g | u]
    gu_re = run(x, w_gu, "DEFAULT", b_layout="NK")                       # recompute alternative
    out = run(h, wd, "DEFAULT", b_layout="NK")
    # backward
    dgu = torch.empty((m, 2 * idim), dtype=torch.bfloat16, device=dev)
    run(dout, wd, "DSWIGLU", {"gate": gu[:, :idim], "up": gu[:, idim:]}, b_layout="KN",
        out=dgu[:, :idim], aux_out={"d_up": dgu[:, idim:]})
    dx = run(dgu, w_gu, "DEFAULT", b_layout="KN")                        # M x H, K = 2I
    dw_gu = run(dgu, x, "DEFAULT", b_layout="KN", a_layout="KM")         # 2I x H
    dwd = run(dout, h, "DEFAULT", b_layout="KN", a_layout="KM")          # H x I
    torch.cuda.synchronize()

    # Every output is checked on seeded 128 x 128 tiles spread over all of it, the four corner
    # tiles included (so the last tile-row and tile-column of every kernel are covered), each
    # against the oracle evaluated on exactly the rows and columns the tile needs.
    def tiles(rows, cols, seed):
        return oracle.sample_tiles(rows, cols, count=12, seed=seed)

    for (r0, r1, c0, c1) in tiles(m, idim, 61):
        xr = f64(x[r0:r1])
        g_ref = oracle.matmul(xr, f64(wg[c0:c1]), "NK")
        u_ref = oracle.matmul(xr, f64(wu[c0:c1]), "NK")
        at = f"tile {(r0, c0)}"
        assert_half(f64(gu[r0:r1, c0:c1]), g_ref, "saved g " + at)
        assert_half(f64(gu[r0:r1, idim + c0:idim + c1]), u_ref, "saved u " + at)
        assert_half(f64(gu_re[r0:r1, c0:c1]), g_ref, "recomputed g " + at)
        assert_half(f64(gu_re[r0:r1, idim + c0:idim + c1]), u_ref, "recomputed u " + at)
        assert_half(f64(h[r0:r1, c0:c1]), oracle.swiglu(xr, f64(wg[c0:c1]), f64(wu[c0:c1]))[0], "h " + at)
        # backward on the GPU's own saved g and u
        dg_ref, du_ref, _ = oracle.dswiglu(f64(dout[r0:r1]), f64(wd[:, c0:c1]), f64(gu[r0:r1, c0:c1]),
                                           f64(gu[r0:r1, idim + c0:idim + c1]))
        assert_half(f64(dgu[r0:r1, c0:c1]), dg_ref, "d_gate " + at)
        assert_half(f64(dgu[r0:r1, idim + c0:idim + c1]), du_ref, "d_up " + at)
    for (r0, r1, c0, c1) in tiles(m, hd, 62):
        at = f"tile {(r0, c0)}"
        assert_half(f64(out[r0:r1, c0:c1]), oracle.matmul(f64(h[r0:r1]), f64(wd[c0:c1]), "NK"), "out " + at)
        assert_half(f64(dx[r0:r1, c0:c1]), oracle.matmul(f64(dgu[r0:r1]), f64(w_gu[:, c0:c1]), "KN"),
                    "dx = d_gate Wg + d_up Wu " + at)
    # weight gradients contract over the whole batch: tile (r, c) of [dWg; dWu] is
    # [d_gate | d_up][:, r]^T x[:, c], of dWd dout[:, r]^T h[:, c]
    for (r0, r1, c0, c1) in tiles(2 * idim, hd, 63):
        assert_half(f64(dw_gu[r0:r1, c0:c1]), oracle.matmul(f64(dgu[:, r0:r1]).T, f64(x[:, c0:c1]), "KN"),
                    f"[dWg; dWu] tile {(r0, c0)}")
    for (r0, r1, c0, c1) in tiles(hd, idim, 64):
        assert_half(f64(dwd[r0:r1, c0:c1]), oracle.matmul(f64(dout[:, r0:r1]).T, f64(h[:, c0:c1]), "KN"),
                    f"dWd tile {(r0, c0)}")
    for p in plans:
        p.free()
