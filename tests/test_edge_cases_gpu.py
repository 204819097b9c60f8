"""GPU edge cases of the ReLU epilogs, forced rather than left to random data.

"Forward-pass capabilities in the source" (Fusing Matmul Epilogs with nvmath-python) defines
the relu_aux bit as the sign test of the pre-activation, and "Backward-pass path shown in the
example" masks the backward product with it.  These tests drive the strict predicate's
boundary on the GPU:

  * forward with A = 0, so that the float32 pre-activation is exactly the bias: bias columns
    hold +0, -0, the smallest subnormals of either sign, +-1e4, the largest finite values,
    NaN and +-inf.  Y and the mask words must equal the oracle's bit for bit: the bit is 0
    for +-0 and NaN and 1 for a positive subnormal, Y is +0 wherever P <= 0 or P is NaN,
    and tail bits past column N-1 are 0.
  * biases that saturate every bit (+-1e4 on ordinary products): all bits set with Y = P,
    or no bit set with Y = +0 everywhere.
  * backward with rows of dY holding +inf, -inf and NaN: masked-out outputs must be exactly
    +0 (a NaN or inf product is dropped, not multiplied by zero), kept ones +-inf / NaN as
    in the oracle, and each bias-gradient column non-finite exactly where the oracle's is.
  * bitwise self-consistency at the square layer's size with one tile configuration:
    relu(Y_BIAS) == Y_RELU_BIAS == Y_RELU_AUX_BIAS.
  * the GELU forward epilogs on the same special pre-activations (A = 0): finite ones follow
    the oracle to one rounding, the non-finite ones the function's limits.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests._gpu import assert_bgrad, assert_half, f64, require_gpu, say, words

pytestmark = pytest.mark.gpu

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}
M, N, K = 300, 200, 192  # ragged against every tile in M and N; N % 32 = 8 leaves tail bits


def special_values(dt):
    fi = torch.finfo(dt)
    sub = torch.tensor(1, dtype=torch.int16).view(dt).item()  # bit pattern 0x0001: the smallest subnormal
    vals = [0.0, -0.0, sub, -sub, 1e4, -1e4, fi.max, -fi.max, float("nan"), float("inf"), float("-inf"),
            fi.smallest_normal, -fi.smallest_normal, 1.5, -1.5]
    t = torch.tensor(vals, dtype=torch.float64).to(dt)
    assert t[2].item() > 0 and t[2].item() < fi.smallest_normal, "smallest subnormal"
    assert (t[0].view(torch.int16).item(), t[1].view(torch.int16).item()) == (0, -32768), "signed zeros"
    return t


def edge_bias(dt, seed):
    """bias of length N: seeded N(0,1) values with every special value placed in a few columns
    (the first tile's columns, a column in the 32-column tail word, and the last column)."""
    g = torch.Generator().manual_seed(seed)
    bias = torch.randn(N, generator=g).to(dt)
    sp = special_values(dt)
    cols = [0, 1, 31, 32, 33, 63, 64, 100, 127, 128, 150, 191, 192, 197, 199]
    for i, c in enumerate(cols):
        bias[c] = sp[i % len(sp)]
    # every special value also at a column of its own index + 40 (a second word, another lane)
    for i in range(len(sp)):
        bias[40 + i] = sp[i]
    return bias


def half_bits(t):
    return t.view(torch.int16).cpu().numpy().astype(np.uint16)


def expected_relu_bits(p_half):
    """Y = P where P > 0 (P NaN fails the test), else +0, as half bit patterns."""
    y = p_half.clone()
    y[~(p_half.float() > 0)] = 0.0
    return half_bits(y)


def run_plan(a, b, epi, ins, layout, cfg, path="fused", **kw):
    import dense_gemm_epilogues_amd as ep
    p = ep.Plan(a, b, epi, ins, b_layout=layout, tile_cfg=cfg, path=path, **kw)
    out, aux = p.execute()
    torch.cuda.synchronize()
    return p, out, aux


CFGS = [0, 8, 9, 10, 11, 12]


@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("dtname", ["f16", "bf16"])
def test_zero_product_special_bias(dtname, layout):
    """A = 0: the pre-activation is the bias itself, so every special value reaches the strict
    predicate unchanged; fused (four tile configurations) and unfused paths."""
    require_gpu()
    dt = DTYPES[dtname]
    dev = torch.device("cuda")
    bias_h = edge_bias(dt, seed=11)
    bias = bias_h.to(dev)
    a = torch.zeros((M, K), dtype=dt, device=dev)
    g = torch.Generator().manual_seed(12)
    b = (torch.randn((K, N) if layout == "KN" else (N, K), generator=g) * K ** -0.5).to(dt).to(dev)
    p_half = bias_h.unsqueeze(0).expand(M, N)           # P = 0 + bias, exactly, on every row
    want_y = expected_relu_bits(p_half)
    p64 = f64(bias_h)[None, :].repeat(M, axis=0)
    want_words = oracle.pack_relu_mask(p64 > 0)          # NaN > 0 is False in float64 too
    nw = want_words.shape[1]
    assert int(want_words[0, -1] >> np.uint32(N % 32)) == 0
    for path, cfgs in (("fused", CFGS), ("unfused", [-1])):
        for cfg in cfgs:
            what = f"{dtname}/{layout}/cfg{cfg}/{path}"
            say(f"case zero-product special bias {what}")
            plans = []
            # BIAS: Y = P exactly (NaN stays NaN); the sign of a zero sum is not part of the
            # definition, so -0 and +0 compare equal here
            p, yb, _ = run_plan(a, b, "BIAS", {"bias": bias}, layout, cfg, path)
            plans.append(p)
            yb_bits = half_bits(yb)
            yb_bits[yb_bits == 0x8000] = 0
            pb = p_half.clone()
            nan = torch.isnan(pb.float()).numpy()
            pb_bits = half_bits(pb)
            pb_bits[pb_bits == 0x8000] = 0
            assert np.array_equal(yb_bits[~nan], pb_bits[~nan]), f"BIAS {what}: Y != bias bitwise"
            assert np.all(np.isnan(f64(yb)[nan])), f"BIAS {what}: NaN bias not propagated"
            # RELU_BIAS and RELU_AUX_BIAS: Y and the mask words bit for bit
            for epi in ("RELU_BIAS", "RELU_AUX_BIAS"):
                p, y, aux = run_plan(a, b, epi, {"bias": bias}, layout, cfg, path)
                plans.append(p)
                got = half_bits(y)
                bad = np.argwhere(got != want_y)
                assert bad.size == 0, (f"{epi} {what}: {len(bad)} outputs differ, first {bad[:4].tolist()} "
                                       f"got {got[tuple(bad[0])]:#06x} want {want_y[tuple(bad[0])]:#06x}")
                if epi == "RELU_AUX_BIAS":
                    gw = words(aux["relu_aux"])
                    diff = np.argwhere(gw != want_words)
                    assert diff.size == 0, (f"relu_aux {what}: words differ at {diff[:4].tolist()}: "
                                            f"got {gw[tuple(diff[0])]:#010x} want {want_words[tuple(diff[0])]:#010x}")
                    assert gw.shape[1] == nw
            # relu(Y_BIAS) == Y_RELU_BIAS (same configuration)
            relu_of_bias = yb.clone()
            relu_of_bias[~(yb.float() > 0)] = 0.0
            assert np.array_equal(half_bits(relu_of_bias), want_y), f"relu(Y_BIAS) {what}"
            for p in plans:
                p.free()


@pytest.mark.parametrize("dtname", ["f16", "bf16"])
def test_saturating_bias(dtname):
    """bias = +1e4 on every column: every bit set (tail bits 0) and Y = P; bias = -1e4: no bit
    set and Y is +0 everywhere (the oracle's +-1e4 pins, on ordinary GEMM products)."""
    require_gpu()
    dt = DTYPES[dtname]
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(21)
    a = torch.randn(M, K, generator=g).to(dt).to(dev)
    b = (torch.randn(K, N, generator=g) * K ** -0.5).to(dt).to(dev)
    nw = (N + 31) // 32
    full = np.full((M, nw), 0xFFFFFFFF, dtype=np.uint32)
    full[:, -1] = (1 << (N % 32)) - 1
    for cfg in CFGS:
        for sign in (1.0, -1.0):
            say(f"case saturating bias {dtname} cfg{cfg} sign {sign}")
            bias = torch.full((N,), sign * 1e4, dtype=dt, device=dev)
            p, y, aux = run_plan(a, b, "RELU_AUX_BIAS", {"bias": bias}, "KN", cfg)
            gw = words(aux["relu_aux"])
            if sign > 0:
                assert np.array_equal(gw, full), f"{dtname} cfg{cfg}: not every bit set"
                ref = oracle.bias_epilog(f64(a), f64(b), f64(bias), "KN")
                assert_half(f64(y), ref, f"{dtname} cfg{cfg} saturated Y = P")
            else:
                assert not gw.any(), f"{dtname} cfg{cfg}: bits set under bias -1e4"
                assert int((y.view(torch.int16) != 0).sum()) == 0, f"{dtname} cfg{cfg}: Y not +0"
            p.free()


def nonfinite_class(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(np.isnan(x), 3, np.where(np.isposinf(x), 1, np.where(np.isneginf(x), 2, 0)))


@pytest.mark.parametrize("bgrad_mode", ["two_pass", "atomic"])
@pytest.mark.parametrize("dtname", ["f16", "bf16"])
def test_drelu_nonfinite_rows(dtname, bgrad_mode):
    """dY rows with +inf, -inf and NaN entries: every masked-out element of dX is exactly +0,
    every kept element of those rows is +-inf / NaN as in the oracle, the other rows agree
    within tolerance, and each bias-gradient column is NaN / +inf / -inf exactly where the
    oracle's is (finite columns within tolerance)."""
    require_gpu()
    dt = DTYPES[dtname]
    dev = torch.device("cuda")
    m, n_out, n_in = 260, 192, 200  # dY m x n_out; W n_in x n_out (given N x K); dX m x n_in
    g = torch.Generator().manual_seed(31)
    dy = torch.randn(m, n_out, generator=g).to(dt)
    w = (torch.randn(n_in, n_out, generator=g) * n_out ** -0.5).to(dt)
    w[w == 0] = 2.0 ** -10  # no exact zero: inf * 0 would be NaN, not +-inf
    rows = {3: float("inf"), 130: float("-inf"), 257: float("nan")}
    for r, v in rows.items():
        dy[r, (7 * r) % n_out] = v
    p_sep = torch.randn(m, n_in, generator=g).numpy()
    mask = oracle.pack_relu_mask(p_sep > 0)
    dxref, bgref = oracle.drelu_bgrad(f64(dy), f64(w), "NK", mask)
    special = np.zeros(m, dtype=bool)
    special[list(rows)] = True
    keep = oracle.unpack_relu_mask(mask, n_in)
    dyd, wd = dy.to(dev), w.to(dev)
    maskd = torch.from_numpy(mask.view(np.int32).copy()).to(dev)
    runs = [("fused", c) for c in CFGS] + ([("unfused", -1)] if bgrad_mode == "two_pass" else [])
    for path, cfg in runs:
        for split in ((0, 3) if path == "fused" and cfg in (9, 10, 11, 12) else (0,)):
            what = f"{dtname}/{bgrad_mode}/cfg{cfg}/{path}/split{split}"
            say(f"case DRELU_BGRAD non-finite dY rows {what}")
            p, dx, aux = run_plan(dyd, wd, "DRELU_BGRAD", {"relu_aux": maskd}, "NK", cfg, path,
                                  bgrad_mode=bgrad_mode, split_k=split)
            dxb = half_bits(dx)
            assert np.all(dxb[~keep] == 0), f"{what}: a masked-out element is not +0"
            got = f64(dx)
            assert np.array_equal(nonfinite_class(got[special]), nonfinite_class(dxref[special])), \
                f"{what}: kept elements of the non-finite rows differ in class from the oracle"
            assert np.array_equal(got[special] == 0, dxref[special] == 0)
            assert_half(got[~special], dxref[~special], f"{what} finite rows")
            bg = aux["drelu_bgrad"].cpu().numpy().astype(np.float64)
            assert np.array_equal(nonfinite_class(bg), nonfinite_class(bgref)), f"{what}: bgrad classes"
            fin = nonfinite_class(bgref) == 0
            assert fin.sum() > 0
            assert_bgrad(bg[fin], bgref[fin], f"{what} finite bgrad columns")
            p.free()


def test_square_relu_family_bitwise():
    """At 4096^3 with the forward's default configuration: relu(Y_BIAS) == Y_RELU_BIAS ==
    Y_RELU_AUX_BIAS bit for bit, and relu_aux is exactly (Y_BIAS's fp32 source > 0), seen here
    as the bits of Y_RELU_AUX_BIAS being set exactly where Y_RELU_AUX_BIAS > 0 or the
    pre-activation rounded to +0 from above."""
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    dev = torch.device("cuda")
    c = W.LINEAR[2]
    inp = W.linear_inputs(c, device=dev)
    x, w, bias = inp["x"], inp["w"], inp["bias"]
    outs = {}
    plans = []
    for epi in ("BIAS", "RELU_BIAS", "RELU_AUX_BIAS"):
        say(f"case square {epi} bitwise family")
        p = ep.Plan(x, w, epi, {"bias": bias}, b_layout="KN")
        assert "tile_cfg=12 " in p.info(), p.info()
        outs[epi] = p.execute()
        plans.append(p)
    torch.cuda.synchronize()
    yb = outs["BIAS"][0]
    relu_b = torch.where(yb > 0, yb, torch.zeros_like(yb))
    assert torch.equal(relu_b.view(torch.int16), outs["RELU_BIAS"][0].view(torch.int16)), "relu(Y_BIAS) != Y_RELU_BIAS"
    assert torch.equal(outs["RELU_BIAS"][0].view(torch.int16), outs["RELU_AUX_BIAS"][0].view(torch.int16)), \
        "Y_RELU_BIAS != Y_RELU_AUX_BIAS"
    ya = outs["RELU_AUX_BIAS"][0]
    wd = outs["RELU_AUX_BIAS"][1]["relu_aux"]
    sh = torch.arange(32, device=dev, dtype=torch.int32)
    bits = ((wd.unsqueeze(-1) >> sh) & 1).reshape(c.m, -1)[:, :c.n].bool()
    assert not bool((ya > 0)[~bits].any()), "positive output without its mask bit"
    assert not bool((yb > 0)[~bits].any()), "positive Y_BIAS without its mask bit"
    # a set bit with Y = +0 needs a positive pre-activation that rounds to +0, which Y_BIAS shows too
    assert torch.equal(bits & ~(ya > 0), bits & (yb.view(torch.int16) == 0)), "mask bits against Y_BIAS"
    for p in plans:
        p.free()


@pytest.mark.parametrize("dtname", ["f16", "bf16"])
def test_gelu_special_preactivations(dtname):
    """GELU_BIAS and GELU_AUX_BIAS with A = 0, so that the pre-activation P is the bias exactly
    (the hotdry.top post names GELU_BIAS; the exact form t Phi(t) is this library's reading).
    Finite special values (signed zeros, subnormals, +-1e4, +-largest finite, +-1.5) follow
    the oracle's gelu to one rounding of the element type; the non-finite ones follow the
    function's limits, which the oracle's product form t (1 + erf(t / sqrt 2)) / 2 leaves
    undefined at -inf: GELU(+inf) = +inf, GELU(-inf) = 0, GELU(NaN) = NaN.  GELU_AUX_BIAS's
    saved pre-activation is P bit for bit."""
    require_gpu()
    dt = DTYPES[dtname]
    dev = torch.device("cuda")
    fi = torch.finfo(dt)
    sub = torch.tensor(1, dtype=torch.int16).view(dt).item()
    bias_h = edge_bias(dt, seed=13)
    bias = bias_h.to(dev)
    a = torch.zeros((M, K), dtype=dt, device=dev)
    g = torch.Generator().manual_seed(14)
    b = (torch.randn((K, N), generator=g) * K ** -0.5).to(dt).to(dev)
    p64 = f64(bias_h)
    fin = np.isfinite(p64)
    want = np.zeros(N)
    want[fin] = oracle.gelu(p64[fin])
    want[p64 == np.inf] = np.inf
    want[p64 == -np.inf] = 0.0
    nan = np.isnan(p64)
    # one rounding to the element type, plus the device Phi's error (far below it)
    rel = 2.0 ** -7 if dt == torch.bfloat16 else 2.0 ** -10
    for path, cfgs in (("fused", [0, 11, 12]), ("unfused", [-1])):
        for cfg in cfgs:
            for epi in ("GELU_BIAS", "GELU_AUX_BIAS"):
                what = f"{epi} {dtname}/cfg{cfg}/{path}"
                say(f"case GELU special pre-activations {what}")
                p, y, aux = run_plan(a, b, epi, {"bias": bias}, "KN", cfg, path)
                got = f64(y)
                assert np.all(np.isnan(got[:, nan])), f"{what}: GELU(NaN) is not NaN"
                ok = ~nan
                err = np.abs(got[:, ok] - want[None, ok])
                lim = rel * np.abs(want[None, ok]) + 2 * sub
                inf_ok = np.isinf(want[None, ok]) & (got[:, ok] == want[None, ok])
                bad = np.argwhere(~((err <= lim) | inf_ok))
                assert bad.size == 0, (f"{what}: {len(bad)} outputs off, first column "
                                       f"{np.flatnonzero(ok)[bad[0][1]]}: P = {p64[ok][bad[0][1]]!r}, "
                                       f"got {got[:, ok][tuple(bad[0])]!r}, want {want[ok][bad[0][1]]!r}")
                if epi == "GELU_AUX_BIAS":
                    pa = aux["gelu_aux"]
                    # (0 + -0 is +0: the sign of a zero sum is not part of the definition)
                    pb = half_bits(bias_h.unsqueeze(0).expand(M, N).contiguous())
                    pg = half_bits(pa)
                    pb[pb == 0x8000] = 0
                    pg[pg == 0x8000] = 0
                    same = (pg == pb) | (np.isnan(f64(pa)) & nan[None, :])
                    assert same.all(), f"{what}: saved pre-activation differs from P"
                p.free()


@pytest.mark.parametrize("path", ["fused", "unfused"])
def test_dswiglu_special_gate_up(path):
    """GEMM + dSwiGLU (gemm_swiglu_mlp_fusion.py docstring; the derivative is this library's
    reading of h = silu(g) u) with special saved pre-activations: gate columns holding +-0, a
    subnormal, +-1.5, -100 (where the logistic function underflows to 0 in fp32), +-1e4, the
    largest finite values, +-inf and NaN; up columns holding 0, +-inf and NaN.  Where the
    oracle's float64 value, rounded to bf16, is NaN or infinite the GPU's must be the same
    (NaN, or the same infinity); elsewhere the output tolerance holds."""
    require_gpu()
    dt = torch.bfloat16
    dev = torch.device("cuda")
    fi = torch.finfo(dt)
    sub = torch.tensor(1, dtype=torch.int16).view(dt).item()
    g = torch.Generator().manual_seed(15)
    m, n, k = M, N, K
    dout = torch.randn((m, k), generator=g).to(dt)
    wd = (torch.randn((k, n), generator=g) * k ** -0.5).to(dt)
    gate = (torch.randn((m, n), generator=g) * 2).to(dt)
    up = torch.randn((m, n), generator=g).to(dt)
    gvals = [0.0, -0.0, sub, 1.5, -1.5, -100.0, 1e4, -1e4, fi.max, -fi.max, float("inf"), float("-inf"), float("nan")]
    for i, v in enumerate(gvals):  # a column each, in the first tile and in the ragged last one
        gate[:, 3 + i] = v
        gate[:, n - 1 - i] = v
    for i, v in enumerate([0.0, float("inf"), float("-inf"), float("nan")]):
        up[:, 40 + i] = v
        up[:, 60 + i] = v
        gate[:, 60 + i] = gvals[6 + i]  # next to gates of 1e4, -1e4, +max, -max
    d_gate_ref, d_up_ref, _ = oracle.dswiglu(f64(dout), f64(wd), f64(gate), f64(up))
    plans = []
    cfgs = [-1, 0, 11, 12] if path == "fused" else [-1]
    for cfg in cfgs:
        what = f"DSWIGLU special gate/up cfg{cfg}/{path}"
        say(f"case {what}")
        p, dg, aux = run_plan(dout.to(dev), wd.to(dev), "DSWIGLU", {"gate": gate.to(dev), "up": up.to(dev)}, "KN",
                              cfg, path)
        plans.append(p)
        for name, got_t, ref in (("d_gate", dg, d_gate_ref), ("d_up", aux["d_up"], d_up_ref)):
            got = f64(got_t)
            with np.errstate(invalid="ignore", over="ignore"):
                rounded = torch.from_numpy(ref).to(dt).double().numpy()  # ref as bf16: beyond its range -> inf
            nonfin = ~np.isfinite(rounded)
            both_nan = np.isnan(rounded) & np.isnan(got)
            same_inf = np.isinf(rounded) & (got == rounded)
            bad = np.argwhere(nonfin & ~(both_nan | same_inf))
            assert bad.size == 0, (f"{what} {name}: {len(bad)} non-finite outputs differ, first {bad[0].tolist()}: "
                                   f"got {got[tuple(bad[0])]!r}, want {rounded[tuple(bad[0])]!r}, "
                                   f"gate {float(gate[tuple(bad[0])])!r}, up {float(up[tuple(bad[0])])!r}")
            bad = np.argwhere(~nonfin & ~np.isfinite(got))
            assert bad.size == 0, f"{what} {name}: non-finite where the oracle is finite, first {bad[0].tolist()}"
            fin = ~nonfin
            rms = float(np.sqrt(np.mean(ref[fin] ** 2)))
            err = np.abs(got[fin] - ref[fin])
            assert np.all(err <= 2e-2 * (np.abs(ref[fin]) + rms)), f"{what} {name}: finite outputs off, max err {err.max()}"
    for p in plans:
        p.free()
