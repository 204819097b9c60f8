"""GPU parity at the largest sizes the C ABI accepts: every leading dimension at its maximum
(ld < 2^22 elements, ld_aux < 2^22 words), and M = 2^31 - 1 rows.

The kernels address a tile's rows with 32-bit offsets from a per-tile or per-slab base and
clamp each buffer extent below 2^31 bytes; a 256-row tile at ld = 2^22 - 8 spans 256 * ld * 2
= 2,147,479,552 bytes, just inside that extent.  Each such case keeps every operand at the
maximum row stride (a few GiB per buffer), fills every byte outside the logical matrices
with NaN or a sentinel, and checks the results against the oracle and the padding for stray
writes.  At M = 2^31 - 1 (N = K = 8: 32 GiB per operand) tile and row indices reach the top
of the 32-bit range; the rows repeat a 7-row pattern, so that every one of the 2^31 - 1 output
rows is checked bit for bit against the pattern's rows on the device, those against the
oracle, and the bias gradient against the oracle's pattern rows weighted by how often each
occurs.  At K = 2^31 - 64 (A given K x M, B K x N) the k-offsets reach the top of the 32-bit
range; that case is built so that float32 accumulation is exact (see its test).  (Epilogs as in "Fusing Matmul Epilogs with nvmath-python"; dSwiGLU as in the
gemm_swiglu_mlp_fusion.py docstring.)"""
import numpy as np
import pytest
import torch

import oracle
from tests._gpu import assert_bgrad, assert_half, f64, require_gpu, say, words

pytestmark = pytest.mark.gpu

LD = (1 << 22) - 8        # largest element leading dimension (a multiple of 8 below 2^22)
LD_AUX = (1 << 22) - 1    # largest mask leading dimension, in 32-bit words
M, N, K = 300, 200, 72    # two tile rows (the first a full 256 rows), ragged N and K
SENT16 = 0x7A5A           # a finite fp16 / bf16 bit pattern no kernel writes here by chance
SENT32 = 0x5A5A5A5A


def strided(rows, cols, ld, dt, dev, fill):
    """a rows x cols view with row stride ld into a buffer filled with `fill`, and the buffer"""
    buf = torch.full((rows, ld), fill, dtype=dt, device=dev)
    return buf[:, :cols], buf


def put(view, src):
    view.copy_(src.to(view.device))
    return view


def randn(shape, seed, scale, dt):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dt)


def untouched16(buf, cols):
    return bool((buf[:, cols:].view(torch.int16) == SENT16).all().item())


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def require_free(gib):
    """skip unless the device has `gib` GiB free (the 2^31-row and 2^31-deep cases hold two or
    three 32 GiB operands; an MI355X has 288 GB)"""
    free()
    if torch.cuda.mem_get_info()[0] < gib << 30:
        pytest.skip(f"needs {gib} GiB of free device memory")


@pytest.mark.parametrize("path", ["fused", "unfused"])
def test_relu_aux_bias_at_max_ld(path):
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    dev, dt = torch.device("cuda"), torch.float16
    say(f"case max-ld RELU_AUX_BIAS f16 KN path={path} m={M} n={N} k={K} ld={LD} ld_aux={LD_AUX}")
    x_h, w_h = randn((M, K), 1, 1.0, dt), randn((K, N), 2, K ** -0.5, dt)
    bias_h = randn((N,), 3, 0.1, dt)
    x, _ = strided(M, K, LD, dt, dev, float("nan"))
    w, _ = strided(K, N, LD, dt, dev, float("nan"))
    put(x, x_h), put(w, w_h)
    bias = bias_h.to(dev)
    out, obuf = strided(M, N, LD, torch.int16, dev, SENT16)
    out, obuf = out.view(dt), obuf.view(dt)
    aux, abuf = strided(M, (N + 31) // 32, LD_AUX, torch.int32, dev, SENT32)
    p = ep.Plan(x, w, "RELU_AUX_BIAS", {"bias": bias}, b_layout="KN", out=out, aux_out={"relu_aux": aux}, path=path)
    p.execute()
    torch.cuda.synchronize()
    yref, _, pre = oracle.relu_aux_bias(f64(x_h), f64(w_h), f64(bias_h), "KN")
    assert_half(f64(out.contiguous()), yref, f"max-ld RELU_AUX_BIAS {path} Y")
    got = words(aux.contiguous())
    ok, info = oracle.check_mask(got, pre)
    assert ok, f"max-ld RELU_AUX_BIAS {path} mask: {info}"
    assert untouched16(obuf, N), "a write outside Y"
    assert bool((abuf[:, (N + 31) // 32:] == SENT32).all().item()), "a write outside relu_aux"
    p.free()
    del x, w, out, obuf, aux, abuf
    free()


def test_drelu_bgrad_at_max_ld():
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    dev, dt = torch.device("cuda"), torch.bfloat16
    say(f"case max-ld DRELU_BGRAD bf16 NK m={M} n={N} k={K} ld={LD} ld_aux={LD_AUX}")
    dy_h, w_h = randn((M, K), 4, 1.0, dt), randn((N, K), 5, K ** -0.5, dt)
    mask_h = torch.from_numpy(oracle.pack_relu_mask(randn((M, N), 6, 1.0, torch.float32).numpy() > 0)
                              .view(np.int32).copy())
    dy, _ = strided(M, K, LD, dt, dev, float("nan"))
    w, _ = strided(N, K, LD, dt, dev, float("nan"))
    put(dy, dy_h), put(w, w_h)
    mask, _ = strided(M, mask_h.shape[1], LD_AUX, torch.int32, dev, -1)
    put(mask, mask_h)
    out, obuf = strided(M, N, LD, torch.int16, dev, SENT16)
    out, obuf = out.view(dt), obuf.view(dt)
    for bgrad_mode in ("two_pass", "atomic"):
        p = ep.Plan(dy, w, "DRELU_BGRAD", {"relu_aux": mask}, b_layout="NK", out=out, bgrad_mode=bgrad_mode)
        _, auxo = p.execute()
        torch.cuda.synchronize()
        dref, bref = oracle.drelu_bgrad(f64(dy_h), f64(w_h), "NK", words(mask_h))
        assert_half(f64(out.contiguous()), dref, f"max-ld DRELU_BGRAD {bgrad_mode} dX")
        assert_bgrad(auxo["drelu_bgrad"].cpu().numpy().astype(np.float64), bref, f"max-ld DRELU_BGRAD {bgrad_mode} bgrad")
        assert untouched16(obuf, N), "a write outside dX"
        p.free()
    del dy, w, mask, out, obuf
    free()


@pytest.mark.parametrize("split_k", [1, 2])
def test_transposed_a_at_max_ld(split_k):
    """A given K x M (a weight gradient's activation; M a multiple of 8) at the maximum
    stride, B K x N too."""
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    dev, dt = torch.device("cuda"), torch.float16
    m, k = M - 4, K * 4
    say(f"case max-ld DEFAULT A^T f16 KN m={m} n={N} k={k} ld={LD} split={split_k}")
    at_h, b_h = randn((k, m), 7, 1.0, dt), randn((k, N), 8, k ** -0.5, dt)
    at, _ = strided(k, m, LD, dt, dev, float("nan"))
    b, _ = strided(k, N, LD, dt, dev, float("nan"))
    put(at, at_h), put(b, b_h)
    out, obuf = strided(m, N, LD, torch.int16, dev, SENT16)
    out, obuf = out.view(dt), obuf.view(dt)
    p = ep.Plan(at, b, "DEFAULT", b_layout="KN", out=out, a_layout="KM", split_k=split_k)
    p.execute()
    torch.cuda.synchronize()
    assert_half(f64(out.contiguous()), oracle.matmul(f64(at_h).T, f64(b_h), "KN"), f"max-ld A^T split {split_k}")
    assert untouched16(obuf, N), "a write outside D"
    p.free()
    del at, b, out, obuf
    free()


def test_dswiglu_at_max_ld():
    """dout · Wd with gate, up, d_gate and d_up all at the maximum row stride."""
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    dev, dt = torch.device("cuda"), torch.bfloat16
    say(f"case max-ld DSWIGLU bf16 KN m={M} n={N} k={K} ld={LD}")
    dout_h, wd_h = randn((M, K), 9, 1.0, dt), randn((K, N), 10, K ** -0.5, dt)
    gate_h, up_h = randn((M, N), 11, 1.0, dt), randn((M, N), 12, 1.0, dt)
    dout, _ = strided(M, K, LD, dt, dev, float("nan"))
    wd, _ = strided(K, N, LD, dt, dev, float("nan"))
    gate, _ = strided(M, N, LD, dt, dev, float("nan"))
    up, _ = strided(M, N, LD, dt, dev, float("nan"))
    for v, h in ((dout, dout_h), (wd, wd_h), (gate, gate_h), (up, up_h)):
        put(v, h)
    dg, dgbuf = strided(M, N, LD, torch.int16, dev, SENT16)
    du, dubuf = strided(M, N, LD, torch.int16, dev, SENT16)
    dg, dgbuf, du, dubuf = dg.view(dt), dgbuf.view(dt), du.view(dt), dubuf.view(dt)
    p = ep.Plan(dout, wd, "DSWIGLU", {"gate": gate, "up": up}, b_layout="KN", out=dg, aux_out={"d_up": du})
    p.execute()
    torch.cuda.synchronize()
    dg_ref, du_ref, _ = oracle.dswiglu(f64(dout_h), f64(wd_h), f64(gate_h), f64(up_h), "KN")
    assert_half(f64(dg.contiguous()), dg_ref, "max-ld DSWIGLU d_gate")
    assert_half(f64(du.contiguous()), du_ref, "max-ld DSWIGLU d_up")
    assert untouched16(dgbuf, N) and untouched16(dubuf, N), "a write outside d_gate / d_up"
    p.free()
    del dout, wd, gate, up, dg, dgbuf, du, dubuf
    free()


MMAX = (1 << 31) - 1      # the largest M the C ABI accepts
P = 7                     # period of the rows at MMAX (divides neither 32 nor 256)


def periodic(pattern, rows, dev):
    """rows x c tensor on the device whose row r is pattern[r % len(pattern)]"""
    reps = -(-rows // pattern.shape[0])
    return pattern.to(dev).repeat(reps, 1)[:rows]


def rows_repeat(t):
    """every row of t (M x c, c * elem_size a multiple of 8 bytes) equals row r % P, bit for bit"""
    v = t.view(torch.int64) if t.element_size() * t.shape[1] % 8 == 0 else t.view(torch.int32)
    full = (v.shape[0] // P) * P
    ok = bool((v[:full].view(-1, P, v.shape[1]) == v[:P].unsqueeze(0)).all().item())
    return ok and bool((v[full:] == v[:v.shape[0] - full]).all().item())


def counts():
    """how many of the MMAX rows repeat each pattern row"""
    c = np.full(P, MMAX // P, dtype=np.float64)
    c[:MMAX % P] += 1
    return c


@pytest.mark.parametrize("path", ["fused", "unfused"])
def test_relu_aux_bias_at_max_m(path):
    require_gpu()
    require_free(90)
    import dense_gemm_epilogues_amd as ep
    dev, dt = torch.device("cuda"), torch.float16
    n = k = 8
    say(f"case max-m RELU_AUX_BIAS f16 KN path={path} m={MMAX} n={n} k={k}")
    pat_h, w_h, bias_h = randn((P, k), 21, 1.0, dt), randn((k, n), 22, k ** -0.5, dt), randn((n,), 23, 0.1, dt)
    x = periodic(pat_h, MMAX, dev)
    w, bias = w_h.to(dev), bias_h.to(dev)
    p = ep.Plan(x, w, "RELU_AUX_BIAS", {"bias": bias}, b_layout="KN", path=path)
    y, aux = p.execute()
    torch.cuda.synchronize()
    del x
    yref, _, pre = oracle.relu_aux_bias(f64(pat_h), f64(w_h), f64(bias_h), "KN")
    assert_half(f64(y[:P].contiguous()), yref, f"max-m RELU_AUX_BIAS {path} pattern rows")
    ok, info = oracle.check_mask(words(aux["relu_aux"][:P].contiguous()), pre)
    assert ok, f"max-m RELU_AUX_BIAS {path} mask: {info}"
    assert rows_repeat(y), "an output row differs from its pattern row"
    assert rows_repeat(aux["relu_aux"]), "a mask row differs from its pattern row"
    p.free()
    del y, aux, p
    free()


def test_drelu_bgrad_at_max_m():
    require_gpu()
    require_free(90)
    import dense_gemm_epilogues_amd as ep
    dev, dt = torch.device("cuda"), torch.bfloat16
    n = k = 8
    say(f"case max-m DRELU_BGRAD bf16 NK m={MMAX} n={n} k={k}")
    dy_pat, w_h = randn((P, k), 24, 1.0, dt), randn((n, k), 25, k ** -0.5, dt)
    mask_pat = torch.from_numpy(oracle.pack_relu_mask(randn((P, n), 26, 1.0, torch.float32).numpy() > 0)
                                .view(np.int32).copy())
    dy = periodic(dy_pat, MMAX, dev)
    mask = periodic(mask_pat, MMAX, dev)
    p = ep.Plan(dy, w_h.to(dev), "DRELU_BGRAD", {"relu_aux": mask}, b_layout="NK")
    dx, auxo = p.execute()
    torch.cuda.synchronize()
    del dy, mask
    dref, _ = oracle.drelu_bgrad(f64(dy_pat), f64(w_h), "NK", words(mask_pat))
    assert_half(f64(dx[:P].contiguous()), dref, "max-m DRELU_BGRAD pattern rows")
    assert rows_repeat(dx), "a dX row differs from its pattern row"
    # over 8.4 million partials a plain float32 second pass drifts by about 1.3e-3 relative on
    # this input (a CPU emulation of its order); the compensated one must stay within 1e-4
    ok, info = oracle.check_bgrad(auxo["drelu_bgrad"].cpu().numpy().astype(np.float64), counts() @ dref, rel_tol=1e-4)
    say(f"max-m DRELU_BGRAD bgrad {info}")
    assert ok, f"max-m DRELU_BGRAD bgrad: {info}"
    p.free()
    del dx, auxo, p
    free()


KMAX = (1 << 31) - 64     # the largest K the C ABI accepts


def test_transposed_a_at_max_k():
    """K = 2^31 - 64 with A given K x M and B K x N (M = N = 8, 32 GiB per operand; the plan
    splits the one tile's K range 8 ways).  The rows of A and B repeat a 6-row pattern of
    -1 / 0 / 1 entries whose second half negates A's first half and repeats B's, so every run
    of whole periods sums to exactly zero, every partial sum is a small integer (exact in
    float32 whatever the order and the split), and the product is the sum over the pattern's
    first K mod 6 rows: the result must equal the oracle's bit for bit."""
    require_gpu()
    require_free(70)
    import dense_gemm_epilogues_amd as ep
    dev, dt = torch.device("cuda"), torch.float16
    m = n = 8
    say(f"case max-k DEFAULT A^T f16 KN m={m} n={n} k={KMAX}")
    g = torch.Generator().manual_seed(31)
    a3 = torch.randint(-1, 2, (3, m), generator=g).to(dt)
    b3 = torch.randint(-1, 2, (3, n), generator=g).to(dt)
    a_pat, b_pat = torch.cat([a3, -a3]), torch.cat([b3, b3])
    at, b = periodic(a_pat, KMAX, dev), periodic(b_pat, KMAX, dev)
    p = ep.Plan(at, b, "DEFAULT", b_layout="KN", a_layout="KM")
    assert "splits=8" in p.info(), p.info()
    y, _ = p.execute()
    torch.cuda.synchronize()
    r = KMAX % 6
    ref = oracle.matmul(f64(a_pat[:r]).T, f64(b_pat[:r]), "KN")
    assert np.abs(ref).max() > 0, "the expected product is not all zeros"
    assert np.array_equal(f64(y.contiguous()), ref), (f64(y.contiguous()), ref)
    p.free()
    del at, b, y, p
    free()


NMAX = (1 << 22) - 8      # the widest N: ldd >= N and every leading dimension is below 2^22


def test_relu_aux_bias_at_max_n():
    """N = 2^22 - 8 output columns (16384 column tiles, 131072 mask words per row) against the
    oracle in full."""
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    dev, dt = torch.device("cuda"), torch.float16
    m, k = 8, 24
    say(f"case max-n RELU_AUX_BIAS f16 KN m={m} n={NMAX} k={k}")
    x_h, w_h, bias_h = randn((m, k), 41, 1.0, dt), randn((k, NMAX), 42, k ** -0.5, dt), randn((NMAX,), 43, 0.1, dt)
    p = ep.Plan(x_h.to(dev), w_h.to(dev), "RELU_AUX_BIAS", {"bias": bias_h.to(dev)}, b_layout="KN")
    y, aux = p.execute()
    torch.cuda.synchronize()
    yref, _, pre = oracle.relu_aux_bias(f64(x_h), f64(w_h), f64(bias_h), "KN")
    assert_half(f64(y), yref, "max-n RELU_AUX_BIAS Y")
    ok, info = oracle.check_mask(words(aux["relu_aux"]), pre)
    assert ok, f"max-n RELU_AUX_BIAS mask: {info}"
    p.free()
    del y, aux, p
    free()


def test_drelu_bgrad_at_max_n():
    """DRELU_BGRAD over N = 2^22 - 8 columns (B given N x K): dX and every bias-gradient column
    against the oracle."""
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    dev, dt = torch.device("cuda"), torch.bfloat16
    m, k = 16, 16
    say(f"case max-n DRELU_BGRAD bf16 NK m={m} n={NMAX} k={k}")
    dy_h, w_h = randn((m, k), 44, 1.0, dt), randn((NMAX, k), 45, k ** -0.5, dt)
    mask_h = torch.from_numpy(oracle.pack_relu_mask(randn((m, NMAX), 46, 1.0, torch.float32).numpy() > 0)
                              .view(np.int32).copy())
    p = ep.Plan(dy_h.to(dev), w_h.to(dev), "DRELU_BGRAD", {"relu_aux": mask_h.to(dev)}, b_layout="NK")
    dx, auxo = p.execute()
    torch.cuda.synchronize()
    dref, bref = oracle.drelu_bgrad(f64(dy_h), f64(w_h), "NK", words(mask_h))
    assert_half(f64(dx), dref, "max-n DRELU_BGRAD dX")
    assert_bgrad(auxo["drelu_bgrad"].cpu().numpy().astype(np.float64), bref, "max-n DRELU_BGRAD bgrad")
    p.free()
    del dx, auxo, p
    free()
