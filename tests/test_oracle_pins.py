"""Pins of the CPU oracle against things other than itself (no GPU needed).

Exact rational brute force, hand-derived fixtures under tests/golden/, closed forms,
special cases that reduce to textbook results, and finite differences.  A few tests
plant a plausible mistake in a copy of an oracle function and check that a pin
catches it.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import core
from tests import _brute

RNG = np.random.default_rng(12345)


def f16(shape, scale=1.0, rng=RNG):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ GEMM (O1)
@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (2, 3, 4), (5, 7, 3), (8, 16, 8), (3, 1, 9)])
def test_matmul_exact_bruteforce(m, n, k, layout):
    a = f16((m, k))
    b = f16((k, n) if layout == "KN" else (n, k))
    got = oracle.matmul(oracle.decode_f16(a), oracle.decode_f16(b), layout)
    exact = _brute.exact_matmul(a.tolist(), b.tolist(), layout)
    bk = b.astype(np.float64) if layout == "KN" else b.astype(np.float64).T
    absprod = np.abs(a.astype(np.float64)) @ np.abs(bk)
    for i in range(m):
        for j in range(n):
            err = abs(Fraction(got[i, j]) - exact[i][j])
            assert err <= Fraction(k * 2.0 ** -52) * Fraction(absprod[i, j]) + Fraction(0)


def test_matmul_exact_config1_shape():
    """All 262,144 multiply-adds of the tiny linear layer (32x64x128) exactly."""
    a = f16((32, 128))
    b = f16((128, 64), 1.0)
    got = oracle.matmul(oracle.decode_f16(a), oracle.decode_f16(b), "KN")
    exact = _brute.exact_matmul(a.tolist(), b.tolist(), "KN")
    absprod = np.abs(a.astype(np.float64)) @ np.abs(b.astype(np.float64))
    err = np.array([[float(abs(Fraction(got[i, j]) - exact[i][j])) for j in range(64)] for i in range(32)])
    assert np.all(err <= 128 * 2.0 ** -52 * absprod)


def test_layouts_are_transposes():
    a = f16((6, 10))
    b = f16((10, 4))
    za = oracle.matmul(a, b, "KN")
    zb = oracle.matmul(a, np.ascontiguousarray(b.T), "NK")
    assert np.array_equal(za, zb)
    with pytest.raises(ValueError):
        oracle.matmul(a, b, "NN")


# ------------------------------------------------------------------ decoding
def test_decode_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x0000, 0x8000, 0x7F80, 0x0001, 0x4049], dtype=np.uint16)
    got = oracle.decode_bf16_bits(bits)
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 0.5 and got[3] == 0.0
    assert got[4] == 0.0 and math.copysign(1.0, got[4]) == -1.0
    assert got[5] == math.inf
    assert got[6] == 2.0 ** -133
    assert got[7] == 3.140625
    # against torch's own bfloat16 conversion (an independent library routine)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, t)


# ------------------------------------------------------------------ epilog fixtures
@pytest.mark.parametrize("layout", ["KN", "NK"])
def test_relu_aux_bias_golden(golden_dir, layout):
    g = load(golden_dir, "relu_aux_bias_2x2x3.json")
    b = np.array(g["b_kn"], dtype=np.float64)
    if layout == "NK":
        b = np.ascontiguousarray(b.T)
    y, words, p = oracle.relu_aux_bias(np.array(g["a"], float), b, np.array(g["bias"], float), layout)
    assert np.array_equal(p, np.array(g["p"], float))
    assert np.array_equal(y, np.array(g["y"], float))
    assert np.array_equal(words, np.array(g["relu_aux"], dtype=np.uint32))
    assert np.array_equal(oracle.relu_bias(np.array(g["a"], float), b, np.array(g["bias"], float), layout), y)


def test_mask_layout_golden(golden_dir):
    g = load(golden_dir, "relu_mask_layout_2x40.json")
    n = g["n"]
    p = -np.ones((2, n))
    p[0, g["positive_columns_row0"]] = 1.0
    p[0, 5] = 0.0
    p[0, 6] = -0.0
    p[1, :] = 2.0
    words = oracle.pack_relu_mask(p > 0)
    assert np.array_equal(words, np.array(g["relu_aux"], dtype=np.uint32))
    assert np.array_equal(oracle.unpack_relu_mask(words, n), p > 0)


def test_drelu_bgrad_golden(golden_dir):
    g = load(golden_dir, "drelu_bgrad_2x3x2.json")
    dx, bgrad = oracle.drelu_bgrad(np.array(g["dy"], float), np.array(g["w"], float), "NK",
                                   np.array(g["relu_aux_in"], dtype=np.uint32))
    assert np.array_equal(dx, np.array(g["dx"], float))
    assert np.array_equal(bgrad, np.array(g["bgrad"], float))


def test_swiglu_golden(golden_dir):
    g = load(golden_dir, "swiglu_1x2x2.json")
    h, gg, uu = oracle.swiglu(np.array(g["x"], float), np.array(g["wg"], float), np.array(g["wu"], float))
    assert np.array_equal(gg, np.array(g["g"], float))
    assert np.array_equal(uu, np.array(g["u"], float))
    assert np.allclose(h, np.array(g["h"]), rtol=1e-15, atol=1e-16)
    # dh = dout . Wd = [1, 1] with dout = [[1]] and Wd = [[1, 1]]
    d_gate, d_up, dh = oracle.dswiglu(np.array([[1.0]]), np.array([[1.0, 1.0]]), gg, uu)
    assert np.array_equal(dh, np.array(g["dh"], float))
    assert np.allclose(d_gate, np.array(g["d_gate"]), rtol=1e-15, atol=1e-16)
    assert np.allclose(d_up, np.array(g["d_up"]), rtol=1e-15, atol=1e-16)


# ------------------------------------------------------------------ exact brute force of the epilogs
@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("m,n,k", [(3, 5, 4), (4, 33, 6), (7, 70, 5), (2, 64, 3)])
def test_relu_aux_bias_bruteforce(m, n, k, layout):
    a = f16((m, k))
    b = f16((k, n) if layout == "KN" else (n, k))
    bias = f16((n,), 0.5)
    y, words, p = oracle.relu_aux_bias(oracle.decode_f16(a), oracle.decode_f16(b), oracle.decode_f16(bias), layout)
    pe, ye, we = _brute.exact_relu_aux_bias(a.tolist(), b.tolist(), bias.tolist(), layout)
    for i in range(m):
        for j in range(n):
            assert abs(Fraction(p[i, j]) - pe[i][j]) <= Fraction(1, 2 ** 40)
            assert abs(Fraction(y[i, j]) - ye[i][j]) <= Fraction(1, 2 ** 40)
    # bit-exact wherever the exact pre-activation is not within rounding of zero
    safe = np.array([[abs(pe[i][j]) > Fraction(1, 2 ** 30) for j in range(n)] for i in range(m)])
    got_bits = oracle.unpack_relu_mask(words, n)
    want_bits = np.array([[(we[i][j // 32] >> (j % 32)) & 1 for j in range(n)] for i in range(m)], dtype=bool)
    assert np.array_equal(got_bits[safe], want_bits[safe])
    assert words.shape == (m, (n + 31) // 32)


@pytest.mark.parametrize("m,n,k", [(3, 5, 4), (5, 40, 7), (6, 3, 64)])
def test_drelu_bgrad_bruteforce(m, n, k):
    dy = f16((m, k))
    w = f16((n, k))  # N x K operand of the backward GEMM
    words = oracle.pack_relu_mask(RNG.random((m, n)) < 0.5)
    dx, bgrad = oracle.drelu_bgrad(oracle.decode_f16(dy), oracle.decode_f16(w), "NK", words)
    dxe, bge = _brute.exact_drelu_bgrad(dy.tolist(), w.tolist(), words.tolist())
    for i in range(m):
        for j in range(n):
            assert abs(Fraction(dx[i, j]) - dxe[i][j]) <= Fraction(1, 2 ** 40)
    for j in range(n):
        assert abs(Fraction(bgrad[j]) - bge[j]) <= Fraction(1, 2 ** 38)


# ------------------------------------------------------------------ special cases (O2-O5)
def test_bias_zero_is_plain_gemm():
    a, b = f16((9, 12)), f16((12, 7))
    y = oracle.bias_epilog(a, b, np.zeros(7), "KN")
    assert np.array_equal(y, a.astype(np.float64) @ b.astype(np.float64))


def test_identity_a_gives_elementwise_relu():
    k = 16
    b = f16((k, 10))
    bias = f16((10,))
    y = oracle.relu_bias(np.eye(k), b, bias, "KN")
    p = b.astype(np.float64) + bias.astype(np.float64)[None, :]
    assert np.array_equal(y, np.maximum(p, 0.0))


def test_bias_orientation_is_per_column():
    """Adding a bias shifts each output column by its own value (not each row)."""
    a, b = f16((5, 8)), f16((8, 6))
    bias = np.arange(6, dtype=np.float64)
    d = oracle.bias_epilog(a, b, bias, "KN") - oracle.bias_epilog(a, b, np.zeros(6), "KN")
    assert np.allclose(d, np.broadcast_to(bias, (5, 6)))


def test_large_bias_saturates():
    a, b = f16((32, 128)), f16((128, 64))
    assert np.all(oracle.relu_bias(a, b, np.full(64, -1e4), "KN") == 0.0)
    p = oracle.bias_epilog(a, b, np.full(64, 1e4), "KN")
    y, words, _ = oracle.relu_aux_bias(a, b, np.full(64, 1e4), "KN")
    assert np.array_equal(y, p)
    assert np.all(words == 0xFFFFFFFF)


@pytest.mark.parametrize("n", [1, 31, 32, 33, 64, 100])
def test_pack_unpack_roundtrip(n):
    bits = RNG.random((7, n)) < 0.5
    words = oracle.pack_relu_mask(bits, ld_aux=(n + 31) // 32 + 2)
    assert np.array_equal(oracle.unpack_relu_mask(words, n), bits)
    assert np.all(words[:, (n + 31) // 32:] == 0)
    popcount = sum(bin(int(w)).count("1") for w in words.ravel())
    assert popcount == int(bits.sum())
    if n % 32:
        assert np.all(words[:, (n - 1) // 32] >> np.uint32(n % 32) == 0)


def test_relu_invariants():
    a, b, bias = f16((40, 50)), f16((50, 70)), f16((70,))
    y, words, p = oracle.relu_aux_bias(a, b, bias, "KN")
    bits = oracle.unpack_relu_mask(words, 70)
    assert np.all(y >= 0)
    assert np.all(y[~bits] == 0)
    assert np.array_equal(bits, p > 0)


def test_drelu_all_ones_closed_form():
    dy, w = f16((64, 48)), f16((40, 48))
    ones = oracle.pack_relu_mask(np.ones((64, 40), bool))
    dx, bgrad = oracle.drelu_bgrad(dy, w, "NK", ones)
    assert np.allclose(dx, dy.astype(np.float64) @ w.astype(np.float64).T, rtol=0, atol=1e-12)
    cf = oracle.bgrad_all_ones_closed_form(dy, w, "NK")
    assert np.allclose(bgrad, cf, rtol=1e-12, atol=1e-10)
    # the same closed form in the other layout
    cf_kn = oracle.bgrad_all_ones_closed_form(dy, np.ascontiguousarray(w.T), "KN")
    assert np.allclose(cf, cf_kn, rtol=1e-12, atol=1e-12)


def test_drelu_all_zeros_and_linearity():
    dy, w = f16((30, 20)), f16((50, 20))
    zeros = oracle.pack_relu_mask(np.zeros((30, 50), bool))
    dx, bgrad = oracle.drelu_bgrad(dy, w, "NK", zeros)
    assert np.all(dx == 0) and np.all(bgrad == 0)
    m = RNG.random((30, 50)) < 0.5
    _, b1 = oracle.drelu_bgrad(dy, w, "NK", oracle.pack_relu_mask(m))
    _, b2 = oracle.drelu_bgrad(dy, w, "NK", oracle.pack_relu_mask(~m))
    assert np.allclose(b1 + b2, oracle.bgrad_all_ones_closed_form(dy, w, "NK"), rtol=1e-12, atol=1e-10)


# ------------------------------------------------------------------ SiLU / SwiGLU (O6, O8)
def test_sigmoid_silu_identities():
    t = np.linspace(-30, 30, 601)
    s = oracle.sigmoid(t)
    assert oracle.sigmoid(np.array([0.0]))[0] == 0.5
    assert np.allclose(oracle.sigmoid(-t), 1 - s, rtol=0, atol=1e-15)
    assert np.allclose(oracle.silu(-t), oracle.silu(t) - t, rtol=1e-12, atol=1e-12)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.silu_grad(np.array([0.0]))[0] == 0.5
    big = oracle.sigmoid(np.array([-1000.0, 1000.0]))
    assert big[0] == 0.0 and big[1] == 1.0
    assert np.all(np.isfinite(oracle.silu_grad(np.array([-1000.0, 1000.0]))))
    for v in [-7.5, -1.0, -0.1, 0.3, 2.0, 9.0]:
        assert abs(oracle.sigmoid(np.array([v]))[0] - _brute.scalar_sigmoid(v)) < 1e-16


def test_silu_grad_central_differences():
    t = np.linspace(-12, 12, 97)
    h = 1e-5
    fd = (oracle.silu(t + h) - oracle.silu(t - h)) / (2 * h)
    assert np.allclose(oracle.silu_grad(t), fd, rtol=0, atol=1e-9)


def test_swiglu_bruteforce_and_special_cases():
    x, wg, wu = f16((4, 8)), f16((6, 8), 0.3), f16((6, 8), 0.3)
    h, g, u = oracle.swiglu(x, wg, wu)
    ge = _brute.exact_matmul(x.tolist(), wg.tolist(), "NK")
    ue = _brute.exact_matmul(x.tolist(), wu.tolist(), "NK")
    for i in range(4):
        for j in range(6):
            gv, uv = float(ge[i][j]), float(ue[i][j])
            want = gv * _brute.scalar_sigmoid(gv) * uv
            assert abs(h[i, j] - want) <= 1e-14 * (1 + abs(want))
    # Wu = Wg gives silu(g) * g; x = 0 gives 0
    h2, g2, _ = oracle.swiglu(x, wg, wg)
    assert np.allclose(h2, oracle.silu(g2) * g2, rtol=1e-15, atol=0)
    h3, _, _ = oracle.swiglu(np.zeros((3, 8)), wg, wu)
    assert np.all(h3 == 0)


def test_dswiglu_is_the_gradient_of_swiglu():
    """<d_gate, dg> + <d_up, du> equals the directional derivative of sum(dh*silu(g)*u)."""
    rng = np.random.default_rng(7)
    dout, wd = rng.standard_normal((5, 6)), rng.standard_normal((6, 9))
    gate, up = 3 * rng.standard_normal((5, 9)), rng.standard_normal((5, 9))
    d_gate, d_up, dh = oracle.dswiglu(dout, wd, gate, up)
    assert np.allclose(dh, dout @ wd)
    F = lambda g, u: float(np.sum(dh * oracle.silu(g) * u))
    for _ in range(5):
        dg, du = rng.standard_normal((5, 9)), rng.standard_normal((5, 9))
        eps = 1e-6
        fd = (F(gate + eps * dg, up + eps * du) - F(gate - eps * dg, up - eps * du)) / (2 * eps)
        an = float(np.sum(d_gate * dg) + np.sum(d_up * du))
        assert abs(fd - an) <= 1e-6 * (1 + abs(an))


# ------------------------------------------------------------------ comparison helpers
def test_check_half_output_thresholds():
    ref = RNG.standard_normal((64, 64))
    ok, _ = oracle.check_half_output(ref * (1 + 1e-3), ref)
    assert ok
    bad = ref.copy()
    bad[3, 4] += 0.5
    ok, info = oracle.check_half_output(bad, ref)
    assert not ok
    nan = ref.copy()
    nan[0, 0] = np.nan
    assert not oracle.check_half_output(nan, ref)[0]
    assert not oracle.check_half_output(ref * 1.03, ref)[0]


def test_check_mask_band_and_tail():
    p = RNG.standard_normal((16, 40))
    words = oracle.pack_relu_mask(p > 0)
    assert oracle.check_mask(words, p)[0]
    # flip a bit well outside the band: caught
    i, j = np.unravel_index(np.argmax(np.abs(p)), p.shape)
    w2 = words.copy()
    w2[i, j // 32] ^= np.uint32(1 << (j % 32))
    assert not oracle.check_mask(w2, p)[0]
    # flip a bit inside the band: tolerated
    p2 = p.copy()
    p2[2, 3] = 1e-9
    w3 = oracle.pack_relu_mask(p2 > 0)
    w3[2, 0] ^= np.uint32(1 << 3)
    ok, info = oracle.check_mask(w3, p2)
    assert ok and info["differ_in_band"] == 1
    # a stray tail bit is caught
    w4 = words.copy()
    w4[0, 1] |= np.uint32(1 << 9)
    assert not oracle.check_mask(w4, p)[0]


def test_check_bgrad():
    ref = RNG.standard_normal(1000)
    assert oracle.check_bgrad(ref + 1e-4 * RNG.standard_normal(1000), ref)[0]
    assert not oracle.check_bgrad(ref * 1.01, ref)[0]


def test_samplers_cover_corners():
    tiles = oracle.sample_tiles(1000, 600, count=8, seed=3)
    assert (0, 128, 0, 128) in tiles
    assert any(t[1] == 1000 and t[3] == 600 for t in tiles)
    assert all(t[2] % 32 == 0 and 0 <= t[0] < t[1] <= 1000 and t[3] <= 600 for t in tiles)
    cols = oracle.sample_columns(500, count=10, seed=1)
    assert cols[0] == 0 and cols[-1] == 499


# ------------------------------------------------------------------ planted mistakes
def test_pins_catch_planted_mistakes(golden_dir, monkeypatch):
    g = load(golden_dir, "relu_aux_bias_2x2x3.json")
    a, b, bias = np.array(g["a"], float), np.array(g["b_kn"], float), np.array(g["bias"], float)

    # (1) bias applied per row instead of per column
    def bias_rows(a_, b_, bias_, layout):
        z = core.matmul(a_, b_, layout)
        return z + np.resize(bias_, z.shape[0])[:, None]
    monkeypatch.setattr(core, "bias_epilog", bias_rows)
    y, words, p = core.relu_aux_bias(a, b, bias, "KN")
    assert not np.array_equal(p, np.array(g["p"], float))
    monkeypatch.undo()

    # (2) most-significant-bit-first packing
    gm = load(golden_dir, "relu_mask_layout_2x40.json")
    p = -np.ones((2, 40))
    p[0, gm["positive_columns_row0"]] = 1.0
    p[1] = 1.0
    msb_first = oracle.pack_relu_mask((p > 0)[:, ::-1])
    assert not np.array_equal(msb_first, np.array(gm["relu_aux"], dtype=np.uint32))

    # (3) dSwiGLU missing the (1 + g (1 - s)) factor fails the finite-difference pin
    rng = np.random.default_rng(1)
    gate, up, dh = rng.standard_normal((3, 4)), rng.standard_normal((3, 4)), rng.standard_normal((3, 4))
    wrong_dg = dh * up * oracle.sigmoid(gate)
    F = lambda gg: float(np.sum(dh * oracle.silu(gg) * up))
    dg = rng.standard_normal((3, 4))
    fd = (F(gate + 1e-6 * dg) - F(gate - 1e-6 * dg)) / 2e-6
    assert abs(fd - float(np.sum(wrong_dg * dg))) > 1e-3

    # (4) a transposed B operand fails the exact brute force
    a2, b2 = f16((3, 4)), f16((4, 4))
    wrong = oracle.matmul(a2, np.ascontiguousarray(b2.T), "KN")
    exact = _brute.exact_matmul(a2.tolist(), b2.tolist(), "KN")
    assert any(abs(Fraction(wrong[i, j]) - exact[i][j]) > Fraction(1, 2 ** 20) for i in range(3) for j in range(4))

    # (5) the tanh approximation of GELU in place of the exact form fails the GELU fixture
    gg = load(golden_dir, "gelu_aux_bias_dgelu_2x2x2.json")
    tanh_gelu = lambda t: 0.5 * t * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (t + 0.044715 * t ** 3)))
    monkeypatch.setattr(core, "gelu", tanh_gelu)
    y, _ = core.gelu_aux_bias(np.array(gg["x"], float), np.array(gg["w"], float), np.array(gg["bias"], float), "KN")
    assert not np.allclose(y, gg["y"], rtol=0, atol=1e-15)
    monkeypatch.undo()


# ---------------------------------------------------------------------------- GELU
def test_gelu_golden(golden_dir):
    g = load(golden_dir, "gelu_aux_bias_dgelu_2x2x2.json")
    x, w, bias = np.array(g["x"], float), np.array(g["w"], float), np.array(g["bias"], float)
    y, p = oracle.gelu_aux_bias(x, w, bias, "KN")
    assert np.allclose(p, g["p"], rtol=0, atol=1e-15)
    assert np.allclose(y, g["y"], rtol=0, atol=1e-15)
    dx, bg = oracle.dgelu_bgrad(np.array(g["dy"], float), np.array(g["w_bwd"], float), "NK", p)
    assert np.allclose(dx, g["dx"], rtol=0, atol=1e-15)
    assert np.allclose(bg, g["bgrad"], rtol=0, atol=1e-15)


def test_gelu_identities_and_limits():
    t = np.linspace(-8, 8, 321)
    assert oracle.gelu(np.array([0.0]))[0] == 0.0
    assert oracle.gelu_grad(np.array([0.0]))[0] == 0.5
    # erf is odd, so gelu(t) - gelu(-t) = t
    assert np.allclose(oracle.gelu(t) - oracle.gelu(-t), t, rtol=0, atol=1e-14)
    # gelu(t) -> t for large t, -> 0 for very negative t; gelu' -> 1 and 0
    big = oracle.gelu(np.array([40.0, -40.0]))
    assert big[0] == 40.0 and abs(big[1]) < 1e-300
    gb = oracle.gelu_grad(np.array([40.0, -40.0]))
    assert gb[0] == 1.0 and abs(gb[1]) < 1e-300
    # the minimum of gelu: gelu'(t*) = 0 near t* = -0.7518 (Phi(t) = -t phi(t))
    tm = np.linspace(-0.76, -0.74, 2001)
    t_star = tm[np.argmin(np.abs(oracle.gelu_grad(tm)))]
    assert abs(t_star + 0.7518) < 2e-4


def test_gelu_grad_central_differences():
    t = np.linspace(-9, 9, 181)
    h = 1e-5
    fd = (oracle.gelu(t + h) - oracle.gelu(t - h)) / (2 * h)
    assert np.allclose(oracle.gelu_grad(t), fd, rtol=0, atol=1e-9)


def test_gelu_aux_bias_special_cases_and_bruteforce():
    x, w, b = f16((5, 8)), f16((8, 6), 0.4), f16((6,), 0.2)
    y, p = oracle.gelu_aux_bias(x, w, b, "KN")
    pe = _brute.exact_matmul(x.tolist(), w.tolist(), "KN")
    for i in range(5):
        for j in range(6):
            assert abs(p[i, j] - (float(pe[i][j]) + float(b[j]))) < 1e-12
    assert np.allclose(y, oracle.gelu(p), rtol=0, atol=0)
    # bias = 0 reduces to gelu of the plain product; the NK layout of W^T gives the same result
    y0, _ = oracle.gelu_aux_bias(x, w, np.zeros(6), "KN")
    assert np.allclose(y0, oracle.gelu(x.astype(float) @ w.astype(float)), rtol=0, atol=1e-15)
    y1, _ = oracle.gelu_aux_bias(x, np.ascontiguousarray(w.T), b, "NK")
    assert np.allclose(y1, y, rtol=0, atol=1e-15)


def test_dgelu_bgrad_closed_form_and_gradient():
    rng = np.random.default_rng(11)
    dy, w = rng.standard_normal((7, 5)), rng.standard_normal((9, 5))   # w: N x K (NK)
    # pre-activation 0 everywhere: gelu'(0) = 1/2, so dX = G / 2 and bgrad = colsum(dY) W^T / 2
    dx, bg = oracle.dgelu_bgrad(dy, w, "NK", np.zeros((7, 9)))
    assert np.allclose(dx, 0.5 * dy @ w.T, rtol=1e-14, atol=1e-14)
    assert np.allclose(bg, 0.5 * oracle.bgrad_all_ones_closed_form(dy, w, "NK"), rtol=1e-13, atol=1e-13)
    # dX is the gradient of sum(G * gelu(P)) with respect to P
    p = 2 * rng.standard_normal((7, 9))
    dx, bg = oracle.dgelu_bgrad(dy, w, "NK", p)
    g = dy @ w.T
    F = lambda q: float(np.sum(g * oracle.gelu(q)))
    for _ in range(5):
        d = rng.standard_normal((7, 9))
        eps = 1e-6
        fd = (F(p + eps * d) - F(p - eps * d)) / (2 * eps)
        assert abs(fd - float(np.sum(dx * d))) <= 1e-6 * (1 + abs(fd))
    assert np.allclose(bg, dx.sum(axis=0), rtol=0, atol=0)
