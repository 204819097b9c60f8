"""GPU parity on small and ragged shapes: every epilog x dtype x B layout x tile config.

Each case compares the HIP kernel's outputs element by element with the float64 oracle on
the same seeded inputs, and checks that padding around every output (extra columns of
the leading dimension, an extra row, extra mask words, extra bgrad entries) still holds
its sentinel afterwards.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import assert_bgrad, assert_half, assert_mask, f64, require_gpu, say, words

pytestmark = pytest.mark.gpu

EPIS = ["DEFAULT", "BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "DRELU_BGRAD", "SWIGLU", "DSWIGLU",
        "GELU_BIAS", "GELU_AUX_BIAS", "DGELU_BGRAD", "SWIGLU_AUX"]
SHAPES = [(300, 200, 136), (37, 8, 8), (130, 264, 520), (1, 64, 72)]
DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}
SENT16 = -1  # 0xFFFF, a NaN pattern in both half types
SENT32 = -1


def padded(m, n, dtype, dev, pad_cols=8):
    """An m x n view into an (m+1) x (n+pad) buffer filled with a sentinel."""
    buf = torch.full((m + 1, n + pad_cols), SENT16, dtype=torch.int16, device=dev).view(dtype)
    return buf, buf[:m, :n]


def dec(t, dtype):
    return f64(t) if dtype != "np" else t


def make_inputs(epi, dt, layout, m, n, k, seed, dev):
    g = torch.Generator().manual_seed(seed)
    rn = lambda *s, scale=1.0: (torch.randn(*s, generator=g) * scale).to(dt)
    x = rn(m, k)
    b = rn(k, n, scale=k ** -0.5) if layout == "KN" else rn(n, k, scale=k ** -0.5)
    ins = {"a": x, "b": b}
    if epi in ("BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "GELU_BIAS", "GELU_AUX_BIAS"):
        ins["bias"] = rn(n, scale=0.5)
    if epi == "DGELU_BGRAD":
        ins["gaux"] = rn(m, n, scale=1.5)  # a saved pre-activation
    if epi == "DRELU_BGRAD":
        p = torch.randn(m, n, generator=g).numpy()
        ins["mask"] = torch.from_numpy(oracle.pack_relu_mask(p > 0).view(np.int32).copy())
    if epi in ("SWIGLU", "SWIGLU_AUX"):
        ins["b2"] = rn(*b.shape, scale=k ** -0.5)
    if epi == "DSWIGLU":
        ins["gate"] = rn(m, n, scale=1.5)
        ins["up"] = rn(m, n, scale=1.5)
    return {kk: v.to(dev) for kk, v in ins.items()}


K64_ONLY_CFGS = (11, 12)  # configurations that need K to be a multiple of 64


def run_and_check(epi, dtname, layout, m, n, k, cfg, path="fused", seed=0, split_k=0, bgrad_mode="two_pass",
                  autotune=False, split_tail=False):
    import dense_gemm_epilogues_amd as ep
    dev = torch.device("cuda")
    dt = DTYPES[dtname]
    if cfg in K64_ONLY_CFGS and k % 64:
        # refused with a ragged K; the case then runs with K rounded up to a multiple of 64
        a = torch.zeros((m, k), dtype=dt, device=dev)
        b = torch.zeros((k, n) if layout == "KN" else (n, k), dtype=dt, device=dev)
        with pytest.raises(ep.EPError, match="EP_ERR_UNSUPPORTED.*multiple of 64"):
            ep.Plan(a, b, "DEFAULT", b_layout=layout, tile_cfg=cfg)
        k = -(-k // 64) * 64
    ins = make_inputs(epi, dt, layout, m, n, k, seed, dev)
    obuf, out = padded(m, n, dt, dev)
    aux_out, epi_in = {}, {}
    nw = (n + 31) // 32
    if epi in ("BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "GELU_BIAS", "GELU_AUX_BIAS"):
        epi_in["bias"] = ins["bias"]
    if epi == "GELU_AUX_BIAS":
        gabuf, gaview = padded(m, n, dt, dev)
        aux_out["gelu_aux"] = gaview
    if epi == "DGELU_BGRAD":
        epi_in["gelu_aux"] = ins["gaux"]
        gbuf = torch.full((n + 4,), float("nan"), dtype=torch.float32, device=dev)
        aux_out["dgelu_bgrad"] = gbuf[:n]
    if epi == "RELU_AUX_BIAS":
        abuf = torch.full((m + 1, nw + 1), SENT32, dtype=torch.int32, device=dev)
        aux_out["relu_aux"] = abuf[:m, :nw]
    if epi == "DRELU_BGRAD":
        epi_in["relu_aux"] = ins["mask"]
        gbuf = torch.full((n + 4,), float("nan"), dtype=torch.float32, device=dev)
        aux_out["drelu_bgrad"] = gbuf[:n]
    if epi in ("SWIGLU", "SWIGLU_AUX"):
        epi_in["b2"] = ins["b2"]
    if epi == "SWIGLU_AUX":
        gubuf, guview = padded(m, 2 * n, dt, dev)
        aux_out["gu"] = guview
    if epi == "DSWIGLU":
        epi_in["gate"], epi_in["up"] = ins["gate"], ins["up"]
        ubuf, uview = padded(m, n, dt, dev)
        aux_out["d_up"] = uview
    say(f"case epi={epi} dt={dtname} layout={layout} m={m} n={n} k={k} cfg={cfg} path={path} split_k={split_k}"
        f" split_tail={split_tail} bgrad_mode={bgrad_mode}")
    p = ep.Plan(ins["a"], ins["b"], epilog=epi, epilog_inputs=epi_in, b_layout=layout, out=out,
                aux_out=aux_out, path=path, tile_cfg=cfg, split_k=split_k, bgrad_mode=bgrad_mode,
                autotune=autotune, split_tail=split_tail)
    if split_k > 1:
        # k-step depth of the tile the plan runs (tile=BMxBNxBK...; the planner's choice when cfg is -1)
        bk = int(p.info().split(" tile=")[1].split("x")[2].rstrip("abcdefghijklmnopqrstuvwxyz_"))
        assert cfg < 0 or bk == (64 if cfg in BK64_CFGS else 32), p.info()
        kt = -(-k // bk)
        per = -(-kt // min(split_k, kt))
        want = -(-kt // per)
        assert f"splits={want} " in p.info(), p.info()
        if split_tail and want > 1:
            # whole rounds of the plan's own grid run unsplit (256 CUs, x2 for two-workgroup tiles)
            info = p.info()
            gm, gn = (int(v) for v in info.split(" grid=")[1].split()[0].split("x"))
            slots = 256 * (2 if "_2wg" in info.split(" tile=")[1].split()[0] else 1)
            assert f"split_tail0={gm * gn // slots * slots} " in info, info
    p.execute()
    torch.cuda.synchronize()

    a64, b64 = f64(ins["a"]), f64(ins["b"])
    what = f"{epi}/{dtname}/{layout}/{m}x{n}x{k}/cfg{cfg}/{path}/split{split_k}"
    if epi == "DEFAULT":
        assert_half(f64(out), oracle.matmul(a64, b64, layout), what)
    elif epi == "BIAS":
        assert_half(f64(out), oracle.bias_epilog(a64, b64, f64(ins["bias"]), layout), what)
    elif epi == "RELU_BIAS":
        assert_half(f64(out), oracle.relu_bias(a64, b64, f64(ins["bias"]), layout), what)
    elif epi == "RELU_AUX_BIAS":
        y, _, pre = oracle.relu_aux_bias(a64, b64, f64(ins["bias"]), layout)
        assert_half(f64(out), y, what)
        assert_mask(words(aux_out["relu_aux"]), pre, what)
        # invariants: bit 0 => Y == 0 exactly; Y >= 0
        bits = oracle.unpack_relu_mask(words(aux_out["relu_aux"]), n)
        yg = f64(out)
        assert np.all(yg >= 0) and np.all(yg[~bits] == 0), what
        ab = words(abuf)
        assert np.all(ab[m, :] == 0xFFFFFFFF) and np.all(ab[:, nw] == 0xFFFFFFFF), f"{what}: mask padding written"
    elif epi == "DRELU_BGRAD":
        dx, bg = oracle.drelu_bgrad(a64, b64, layout, words(ins["mask"]))
        assert_half(f64(out), dx, what)
        assert_bgrad(aux_out["drelu_bgrad"].cpu().numpy(), bg, what)
        assert torch.isnan(gbuf[n:]).all(), f"{what}: bgrad padding written"
    elif epi in ("SWIGLU", "SWIGLU_AUX"):
        h, g, u = oracle.swiglu(a64, b64, f64(ins["b2"]), layout)
        assert_half(f64(out), h, what)
        if epi == "SWIGLU_AUX":
            assert_half(f64(aux_out["gu"][:, :n]), g, what + " gate")
            assert_half(f64(aux_out["gu"][:, n:]), u, what + " up")
            gb = gubuf.view(torch.int16).cpu().numpy()
            assert np.all(gb[m, :] == -1) and np.all(gb[:, 2 * n:] == -1), f"{what}: gu padding written"
    elif epi == "DSWIGLU":
        dg, du, _ = oracle.dswiglu(a64, b64, f64(ins["gate"]), f64(ins["up"]), layout)
        assert_half(f64(out), dg, what)
        assert_half(f64(aux_out["d_up"]), du, what)
        ub = ubuf.view(torch.int16).cpu().numpy()
        assert np.all(ub[m, :] == -1) and np.all(ub[:, n:] == -1), f"{what}: d_up padding written"
    elif epi in ("GELU_BIAS", "GELU_AUX_BIAS"):
        y, pre = oracle.gelu_aux_bias(a64, b64, f64(ins["bias"]), layout)
        assert_half(f64(out), y, what)
        if epi == "GELU_AUX_BIAS":
            assert_half(f64(aux_out["gelu_aux"]), pre, what)
            gb = gabuf.view(torch.int16).cpu().numpy()
            assert np.all(gb[m, :] == -1) and np.all(gb[:, n:] == -1), f"{what}: gelu_aux padding written"
    elif epi == "DGELU_BGRAD":
        dx, bg = oracle.dgelu_bgrad(a64, b64, layout, f64(ins["gaux"]))
        assert_half(f64(out), dx, what)
        assert_bgrad(aux_out["dgelu_bgrad"].cpu().numpy(), bg, what)
        assert torch.isnan(gbuf[n:]).all(), f"{what}: bgrad padding written"
    ob = obuf.view(torch.int16).cpu().numpy()
    assert np.all(ob[m, :] == -1) and np.all(ob[:, n:] == -1), f"{what}: output padding written"
    p.free()


# every tile configuration of the library (9 and 10 issue 16x16x32 MFMAs); those with a
# 128-row B tile cannot hold the gate and up sub-tiles of a K x N dual B operand
NUM_TILE_CFGS = 13
BNT128_CFGS = (1, 2, 6)
BK64_CFGS = (1, 4, 8, 11, 12)  # 64-deep k-steps


@pytest.mark.parametrize("cfg", list(range(NUM_TILE_CFGS)))
@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("dtname", ["f16", "bf16"])
@pytest.mark.parametrize("epi", EPIS)
def test_small_shapes_fused(epi, dtname, layout, cfg):
    require_gpu()
    if epi in ("SWIGLU", "SWIGLU_AUX") and layout == "KN" and cfg in BNT128_CFGS:
        import dense_gemm_epilogues_amd as ep
        dev = torch.device("cuda")
        a = torch.zeros((64, 64), dtype=DTYPES[dtname], device=dev)
        with pytest.raises(ep.EPError, match="EP_ERR_UNSUPPORTED"):
            ep.Plan(a, a, epi, {"b2": a}, b_layout="KN", tile_cfg=cfg)
        return
    for (m, n, k) in SHAPES:
        run_and_check(epi, dtname, layout, m, n, k, cfg)


@pytest.mark.parametrize("splits", [2, 3, 4])
@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("epi", EPIS)
def test_split_k(epi, layout, splits):
    """K split over 2-4 workgroups per tile (fp32 partials, then a fixup launch that sums them
    and runs the epilog): every epilog, both dtypes, five tile configurations, a K that
    divides unevenly and a K too short for the requested number of ranges.  Configuration 8
    (register-staged, 64-deep k-steps) is the planner's choice for N x K GEMMs under one round
    of tiles, where the split model splits long K ranges."""
    require_gpu()
    for cfg in (0, 1, 6, 8, 9, 10, 11, 12):
        if epi in ("SWIGLU", "SWIGLU_AUX") and layout == "KN" and cfg in BNT128_CFGS:
            continue
        for dtname in ("f16", "bf16"):
            for (m, n, k) in [(300, 200, 520), (130, 264, 136)]:
                run_and_check(epi, dtname, layout, m, n, k, cfg, split_k=splits)


@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("epi", EPIS)
def test_split_tail(epi, layout):
    """Split-K on the last, partly filled round only: 17 x 16 = 272 output tiles on 256 CUs,
    so tiles [0, 256) run whole-K in one launch and the other 16 are split into K ranges whose
    partials a fixup launch sums before the epilog.  Every epilog, both dtypes, the 64-deep
    16x16 configuration (3 and 8 ranges) and a 32x32 one (8 ranges); the two-pass bias
    gradient sums column partials written by both launches' epilogs.  Also 8 ranges over
    every tile of a small grid (the fixup's largest sum)."""
    require_gpu()
    n = 2048 if epi in ("SWIGLU", "SWIGLU_AUX") else 4096
    for dtname, cfg, splits in (("f16", 11, 3), ("bf16", 11, 8), ("bf16", 0, 8)):
        run_and_check(epi, dtname, layout, 4352 - 40, n - 24, 512, cfg, split_k=splits, split_tail=True)
    # the most ranges a plan takes, over every tile of a small grid (one k-step per range)
    run_and_check(epi, "f16", layout, 300, 200, 512, 11, split_k=8)


def test_split_tail_refusals_and_atomic_bgrad():
    """split_tail needs a partly filled last round: a grid under one round and one of whole
    rounds are refused; the atomic bias gradient also works with a split tail."""
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    dev = torch.device("cuda")
    for (m, n) in [(300, 200), (4096, 4096)]:
        a = torch.zeros((m, 64), dtype=torch.float16, device=dev)
        b = torch.zeros((64, n), dtype=torch.float16, device=dev)
        with pytest.raises(ep.EPError, match="EP_ERR_UNSUPPORTED.*split_tail"):
            ep.Plan(a, b, "DEFAULT", b_layout="KN", tile_cfg=11, split_k=2, split_tail=True)
    run_and_check("DRELU_BGRAD", "f16", "NK", 4352, 4096, 512, 11, split_k=4, split_tail=True, bgrad_mode="atomic")


@pytest.mark.parametrize("cfg", [9, 10, 11, 12])
@pytest.mark.parametrize("layout", ["KN", "NK"])
def test_kstep_pair_k_lengths(layout, cfg):
    """The 16x16 configurations' load schedules over many K lengths.  Configurations 9 and 10
    load k-steps in pairs (k-steps kt+3 and kt+4 issued from each odd k-step kt on, the prologue
    starting the pair (2, 3)); configuration 11 loads k-step kt+2 right after k-step kt's
    barrier into a 2-stage ring.  K from one 32-deep k-step to 18, even and odd counts, ragged
    last k-steps, and split-K ranges of either parity."""
    require_gpu()
    for k in (32, 64, 96, 128, 160, 192, 224, 256, 288, 320, 544, 576, 40, 104):
        run_and_check("DEFAULT", "f16", layout, 260, 296, k, cfg)
    for epi in ("RELU_AUX_BIAS", "DRELU_BGRAD", "DSWIGLU", "SWIGLU", "SWIGLU_AUX"):
        for k in (64, 256):
            run_and_check(epi, "bf16", layout, 260, 296, k, cfg)
    for splits in (2, 3):
        for k in (512, 1024, 608):
            run_and_check("DEFAULT", "f16", layout, 260, 296, k, cfg, split_k=splits)


@pytest.mark.parametrize("epi", EPIS)
def test_autotune(epi):
    """Plan-time tuning picks some (tile, split) pair; the tuned plan must still be exact, and a
    second plan of the same problem reuses the cached choice."""
    require_gpu()
    for layout in ("KN", "NK"):
        run_and_check(epi, "bf16", layout, 300, 200, 520, -1, autotune=True)
        run_and_check(epi, "bf16", layout, 300, 200, 520, -1, autotune=True, seed=1)


@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("dtname", ["f16", "bf16"])
def test_transposed_a(dtname, layout):
    """A given K x M (the GEMM uses its transpose, as a weight gradient X^T dY does), DEFAULT
    epilog: every tile configuration, unsplit and split, with ragged M, N and K tails."""
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    dev = torch.device("cuda")
    dt = DTYPES[dtname]
    for (m, n, k) in [(296, 200, 136), (40, 8, 8), (136, 264, 520), (8, 64, 72), (136, 200, 192), (8, 72, 640)]:
        g = torch.Generator().manual_seed(m + n + k)
        at = (torch.randn(k, m, generator=g)).to(dt).to(dev)          # K x M
        b = (torch.randn(k, n, generator=g) * k ** -0.5).to(dt) if layout == "KN" else \
            (torch.randn(n, k, generator=g) * k ** -0.5).to(dt)
        b = b.to(dev)
        ref = oracle.matmul(f64(at).T, f64(b), layout)
        for cfg in range(NUM_TILE_CFGS):
            if cfg in K64_ONLY_CFGS and k % 64:
                with pytest.raises(ep.EPError, match="EP_ERR_UNSUPPORTED"):
                    ep.Plan(at, b, "DEFAULT", b_layout=layout, tile_cfg=cfg, a_layout="KM")
                continue
            for split in (1, 2):
                obuf, out = padded(m, n, dt, dev)
                say(f"case A^T dt={dtname} layout={layout} m={m} n={n} k={k} cfg={cfg} split={split}")
                p = ep.Plan(at, b, "DEFAULT", b_layout=layout, out=out, tile_cfg=cfg, split_k=split, a_layout="KM")
                p.execute()
                torch.cuda.synchronize()
                assert_half(f64(out), ref, f"A^T {dtname}/{layout}/{m}x{n}x{k}/cfg{cfg}/split{split}")
                ob = obuf.view(torch.int16).cpu().numpy()
                assert np.all(ob[m, :] == -1) and np.all(ob[:, n:] == -1), "output padding written"
                p.free()


@pytest.mark.parametrize("m,n,layout,ld_extra,dual,want_cfg,k", [
    (4096, 4096, "NK", 64, False, 11, 4096),    # K % 64 == 0: 64-deep 16x16x32 k-steps, both layouts
    (4096, 4096, "KN", 0, False, 12, 4096),     # K x N B: with two barriers per k-step
    (16384, 32768, "NK", 64, False, 11, 4096),  # 32 rounds
    (16384, 32768, "NK", 0, False, 11, 4096),   # 32 rounds, B rows 32 KiB apart
    (16384, 32768, "KN", 0, False, 12, 4096),
    (16384, 16384, "KN", 0, False, 11, 8192),   # K x N B, long K over 16 rounds: one barrier
    (2048, 8192, "NK", 0, True, 11, 4096),      # dual-B SwiGLU, N x K weights, 2 rounds
    (2048, 5120, "NK", 0, False, 11, 4096),     # single B, N x K, 160 tiles (under one round)
    (2048, 5120, "KN", 0, False, 12, 4096),
    (2048, 5120, "NK", 0, False, 8, 4072),      # ... with K % 64 != 0: register-staged
    (4096, 4096, "NK", 64, False, 10, 4064),    # K % 64 != 0: 32-deep, rows kept whole for N x K B
    (4096, 4096, "KN", 0, False, 9, 4064),      # ... chunks spread for K x N B
])
def test_planner_tile_choice(m, n, layout, ld_extra, dual, want_cfg, k):
    """The planner's default tile configuration at full-chip shapes (256 CUs), B rows 16384
    (+ ld_extra) elements apart when B is N x K; the result is checked against the oracle on
    sampled rows and columns (the dual-B case on h = silu(x Wg^T) * (x Wu^T))."""
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    dev = torch.device("cuda")
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the expected choices assume 256 CUs")
    g = torch.Generator(device=dev)
    g.manual_seed(m + n + ld_extra)
    a = torch.randn(m, k, device=dev, generator=g).half()

    def b_of():
        if layout == "NK":
            return (torch.randn(n, 16384 + ld_extra, device=dev, generator=g) * k ** -0.5).half()[:, :k]
        return (torch.randn(k, n, device=dev, generator=g) * k ** -0.5).half()
    b = b_of()
    say(f"case planner choice layout={layout} dual={dual} ldb={b.stride(0)} {m}x{n}x{k}")
    rows = torch.tensor(np.r_[0:32, m // 2 - 8:m // 2 + 24, m - 32:m], device=dev)
    cols = torch.tensor(np.r_[0:64, n // 2:n // 2 + 64, n - 64:n], device=dev)
    if dual:
        b2 = b_of()
        p = ep.Plan(a, b, "SWIGLU", {"b2": b2}, b_layout=layout)
        assert f"tile_cfg={want_cfg} " in p.info(), p.info()
        out, _ = p.execute()
        torch.cuda.synchronize()
        ref = oracle.swiglu(f64(a[rows]), f64(b[cols]), f64(b2[cols]), layout)[0]
    else:
        p = ep.Plan(a, b, "DEFAULT", b_layout=layout)
        assert f"tile_cfg={want_cfg} " in p.info(), p.info()
        out, _ = p.execute()
        torch.cuda.synchronize()
        bsel = b[cols] if layout == "NK" else b[:, cols]
        ref = oracle.matmul(f64(a[rows]), f64(bsel), layout)
    assert_half(f64(out[rows][:, cols]), ref, f"planner {layout}/{m}x{n}/{ld_extra}/dual={dual}")
    p.free()


@pytest.mark.parametrize("m,n,k,dual,layout,want", [
    (2048, 17408, 5120, False, "KN", "splits=4 split_tail0=512 "),   # dSwiGLU GEMM at M 2048: 2 rounds + 32 tiles
    (2048, 17408, 5120, True, "NK", "splits=3 split_tail0=1024 "),   # dual-B SwiGLU at M 2048: 4 rounds + 64 tiles
    (34816, 5120, 2048, False, "KN", "splits=1 split_tail0=0 "),     # short K: never split
    (16384, 17408, 5120, False, "KN", "splits=1 split_tail0=0 "),    # whole rounds (17)
])
def test_planner_split_tail_choice(m, n, k, dual, layout, want):
    """Grids with a partly filled last round: the planner splits only the last round's tiles
    where its model expects a gain (the SwiGLU-MLP GEMMs at M 2048, K 5120), and nowhere for a
    short K or whole rounds.  Sampled rows and columns against the oracle."""
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    dev = torch.device("cuda")
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the expected choice assumes 256 CUs")
    g = torch.Generator(device=dev)
    g.manual_seed(m + n + k)
    a = torch.randn(m, k, device=dev, generator=g).to(torch.bfloat16)
    shape_b = (n, k) if layout == "NK" else (k, n)
    b = (torch.randn(*shape_b, device=dev, generator=g) * k ** -0.5).to(torch.bfloat16)
    say(f"case planner split tail {m}x{n}x{k} dual={dual} {layout}")
    if dual:
        b2 = (torch.randn(*shape_b, device=dev, generator=g) * k ** -0.5).to(torch.bfloat16)
        p = ep.Plan(a, b, "SWIGLU", {"b2": b2}, b_layout=layout)
    else:
        p = ep.Plan(a, b, "DEFAULT", b_layout=layout)
    info = p.info()
    assert want in info, info
    out, _ = p.execute()
    torch.cuda.synchronize()
    rows = torch.tensor(np.r_[0:32, m // 2 - 8:m // 2 + 24, m - 32:m], device=dev)
    cols = torch.tensor(np.r_[0:64, n // 2:n // 2 + 64, n - 64:n], device=dev)
    bsel = (lambda t: t[cols]) if layout == "NK" else (lambda t: t[:, cols])
    if dual:
        ref = oracle.swiglu(f64(a[rows]), f64(bsel(b)), f64(bsel(b2)), layout)[0]
    else:
        ref = oracle.matmul(f64(a[rows]), f64(bsel(b)), layout)
    assert_half(f64(out[rows][:, cols]), ref, f"planner split tail {info}")
    p.free()


@pytest.mark.parametrize("a_layout,k,want_cfg", [("MK", 34816, 11), ("KM", 34816, 11), ("MK", 34808, 8)])
def test_planner_split_choice(a_layout, k, want_cfg):
    """A long-K GEMM under one round of tiles, B given N x K (the SwiGLU dx GEMM's shape,
    2048 x 5120 x 34816): the planner picks the 64-deep 16x16 configuration 11 with 3 split-K
    ranges over every tile; with K not a multiple of 64 (34808) the register-staged
    configuration 8, also split 3 ways.  Sampled rows and columns against the oracle."""
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    dev = torch.device("cuda")
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the expected choice assumes 256 CUs")
    m, n = 2048, 5120
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    a = torch.randn(m, k, device=dev, generator=g).half()
    if a_layout == "KM":
        a = a.t().contiguous()
    b = (torch.randn(n, k, device=dev, generator=g) * k ** -0.5).half()
    say(f"case planner split choice A {a_layout} {m}x{n}x{k}")
    p = ep.Plan(a, b, "DEFAULT", b_layout="NK", a_layout=a_layout)
    info = p.info()
    assert f"tile_cfg={want_cfg} " in info and "splits=3 " in info and "split_tail0=0 " in info, info
    out, _ = p.execute()
    torch.cuda.synchronize()
    rows = torch.tensor(np.r_[0:32, m // 2 - 8:m // 2 + 24, m - 32:m], device=dev)
    cols = torch.tensor(np.r_[0:64, n // 2:n // 2 + 64, n - 64:n], device=dev)
    am = a if a_layout == "MK" else a.t()
    ref = oracle.matmul(f64(am[rows]), f64(b[cols]), "NK")
    assert_half(f64(out[rows][:, cols]), ref, f"planner split {a_layout} {info}")
    p.free()


def test_split_k_atomic_bgrad():
    require_gpu()
    run_and_check("DRELU_BGRAD", "f16", "NK", 300, 200, 520, 0, split_k=3, bgrad_mode="atomic")


@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("epi", EPIS)
def test_small_shapes_unfused(epi, layout):
    require_gpu()
    for (m, n, k) in SHAPES:
        run_and_check(epi, "f16" if epi not in ("SWIGLU", "DSWIGLU", "SWIGLU_AUX") else "bf16", layout, m, n, k, -1,
                      path="unfused")


@pytest.mark.parametrize("epi", EPIS)
def test_unfused_rows_past_grid_limit(epi):
    """The unfused path's elementwise kernels launch at most 65535 row-blocks and loop over the
    remaining rows: M = 70001 rows (ragged N and K) against the oracle in full."""
    require_gpu()
    run_and_check(epi, "f16" if epi not in ("SWIGLU", "DSWIGLU", "SWIGLU_AUX") else "bf16", "NK", 70001, 72, 40, -1,
                  path="unfused")


@pytest.mark.parametrize("epi", ["DRELU_BGRAD", "DGELU_BGRAD"])
def test_bgrad_over_many_partial_rows(epi):
    """The two-pass bias gradient's second pass splits the partial rows (one per 256-row tile)
    over 16 groups of 8 loads, 64 columns per workgroup: 131 partial rows (more than one pass
    of 128, a ragged last group) and N = 200 (a workgroup with 8 of its 64 columns), against
    the oracle in full."""
    require_gpu()
    run_and_check(epi, "f16", "NK", 131 * 256 - 216, 200, 64, -1)
    run_and_check(epi, "bf16", "KN", 131 * 256 - 216, 200, 72, 8)


def test_tiny_linear_layer_config():
    """The tiny fp16 linear layer: X 32x128, W 128x64, bias 64; backward dY 32x64 masked by a
    separate 32x128 pre-activation's relu_aux."""
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    c = workloads.LINEAR[1]
    inp = workloads.linear_inputs(c)
    p_sep = workloads.randn((c.m, c.k), workloads.seed_of(1, 5), 1.0, torch.float32)
    mask_in = torch.from_numpy(oracle.pack_relu_mask(p_sep.numpy() > 0).view(np.int32).copy())
    dev = torch.device("cuda")
    x, w, bias, dy = (inp[kk].to(dev) for kk in ("x", "w", "bias", "dy"))
    x64, w64, b64, dy64 = f64(x), f64(w), f64(bias), f64(dy)
    p1 = ep.Plan(x, w, "RELU_BIAS", {"bias": bias}, b_layout="KN")
    y1, _ = p1.execute()
    p2 = ep.Plan(x, w, "RELU_AUX_BIAS", {"bias": bias}, b_layout="KN")
    y2, aux = p2.execute()
    p3 = ep.Plan(dy, w, "DRELU_BGRAD", {"relu_aux": mask_in.to(dev)}, b_layout="NK")
    dx, aux3 = p3.execute()
    torch.cuda.synchronize()
    yref, _, pre = oracle.relu_aux_bias(x64, w64, b64, "KN")
    assert_half(f64(y1), yref, "cfg1 RELU_BIAS")
    assert_half(f64(y2), yref, "cfg1 RELU_AUX_BIAS")
    assert torch.equal(y1, y2), "RELU_BIAS and RELU_AUX_BIAS outputs differ"
    assert_mask(words(aux["relu_aux"]), pre, "cfg1 relu_aux")
    dxref, bgref = oracle.drelu_bgrad(dy64, w64, "NK", words(mask_in))
    assert_half(f64(dx), dxref, "cfg1 DRELU_BGRAD dX")
    assert_bgrad(aux3["drelu_bgrad"].cpu().numpy(), bgref, "cfg1 bgrad")
    for p in (p1, p2, p3):
        p.free()


@pytest.mark.parametrize("m,n,k,epi,dtname,layout,a_layout", [
    (65536, 8192, 16384, "RELU_AUX_BIAS", "f16", "KN", "MK"),
    (65536, 16384, 8192, "DRELU_BGRAD", "f16", "NK", "MK"),
    (2048, 17408, 5120, "SWIGLU", "bf16", "NK", "MK"),
    (2048, 17408, 5120, "DSWIGLU", "bf16", "KN", "MK"),
    (2048, 5120, 17408, "DEFAULT", "bf16", "NK", "MK"),
    (34816, 5120, 2048, "DEFAULT", "bf16", "KN", "KM"),
    (4096, 4096, 4096, "GELU_AUX_BIAS", "f16", "KN", "MK"),
    (300, 200, 136, "DGELU_BGRAD", "f16", "NK", "MK"),
])
def test_describe_matches_plan(m, n, k, epi, dtname, layout, a_layout):
    """ep_plan_describe at this device's CU count states exactly the plan ep_plan_ex makes
    (tile configuration, grid, splits, tail split, workspace, kernels)."""
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    dev = torch.device("cuda")
    dt = DTYPES[dtname]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    a = torch.empty((m, k) if a_layout == "MK" else (k, m), dtype=dt, device=dev)
    b = torch.empty((k, n) if layout == "KN" else (n, k), dtype=dt, device=dev)
    ins = {}
    if epi in ("RELU_AUX_BIAS", "GELU_AUX_BIAS"):
        ins["bias"] = torch.empty(n, dtype=dt, device=dev)
    if epi == "DRELU_BGRAD":
        ins["relu_aux"] = torch.empty((m, (n + 31) // 32), dtype=torch.int32, device=dev)
    if epi == "DGELU_BGRAD":
        ins["gelu_aux"] = torch.empty((m, n), dtype=dt, device=dev)
    if epi == "SWIGLU":
        ins["b2"] = torch.empty_like(b)
    if epi == "DSWIGLU":
        ins["gate"], ins["up"] = torch.empty((m, n), dtype=dt, device=dev), torch.empty((m, n), dtype=dt, device=dev)
    p = ep.Plan(a, b, epi, ins or None, b_layout=layout, a_layout=a_layout)
    want = ep.describe_plan(m, n, k, epi, dt, b_layout=layout, a_layout=a_layout, cus=cus)
    say(f"case describe {epi} {m}x{n}x{k}: {want}")
    assert p.info() == want, (p.info(), want)
    p.free()
