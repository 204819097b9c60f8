"""The planner on the host (no GPU): ep_plan_describe returns the plan ep_plan_ex would make on a
device with a given number of compute units, so the planner's choices -- tile configuration,
split-K, the split of the last partly filled round, workspace -- are checked here on the CPU
for the workloads' shapes and for the rules the GPU tests exercise on 256 CUs.  (The plan/
execute split of "Fusing Matmul Epilogs with nvmath-python", "The problem addressed by fused
epilogs": planning is the host-side step.)"""
import re

import pytest
import torch

import dense_gemm_epilogues_amd as ep

BF16, F16 = torch.bfloat16, torch.float16


def fields(info):
    return dict(re.findall(r"(\w+)=(\S+)", info.split(" kernels=")[0]))


@pytest.mark.parametrize("m,n,k,layout,dual,want_cfg", [
    (4096, 4096, 4096, "NK", False, 11),     # K % 64 == 0: 64-deep 16x16x32 k-steps
    (4096, 4096, 4096, "KN", False, 12),     # K x N B: two barriers per k-step
    (16384, 32768, 4096, "NK", False, 11),   # 32 rounds
    (16384, 32768, 4096, "KN", False, 12),
    (16384, 16384, 8192, "KN", False, 11),   # K x N B, long K over 16 rounds: one barrier
    (2048, 8192, 4096, "NK", True, 11),      # dual-B SwiGLU, N x K weights
    (2048, 5120, 4096, "NK", False, 11),     # single B, N x K, 160 tiles (under one round)
    (2048, 5120, 4096, "KN", False, 12),
    (2048, 5120, 4072, "NK", False, 8),      # ... K % 64 != 0: register-staged
    (4096, 4096, 4064, "NK", False, 10),     # K % 64 != 0: 32-deep, rows kept whole for N x K B
    (4096, 4096, 4064, "KN", False, 9),      # ... chunks spread for K x N B
])
def test_tile_choice(m, n, k, layout, dual, want_cfg):
    info = ep.describe_plan(m, n, k, "SWIGLU" if dual else "DEFAULT", F16, b_layout=layout)
    assert fields(info)["tile_cfg"] == str(want_cfg), info


@pytest.mark.parametrize("m,n,k,epi,layout,splits,tail0", [
    (2048, 17408, 5120, "DSWIGLU", "KN", 4, 512),    # dSwiGLU at M 2048: 2 rounds + 32 tiles
    (2048, 17408, 5120, "SWIGLU", "NK", 3, 1024),    # dual-B SwiGLU at M 2048: 4 rounds + 64 tiles
    (34816, 5120, 2048, "DEFAULT", "KN", 1, 0),      # short K: never split
    (16384, 17408, 5120, "DSWIGLU", "KN", 1, 0),     # whole rounds (17)
    (2048, 5120, 17408, "DEFAULT", "NK", 3, 0),      # the 160-tile down GEMM: every tile, 3 ranges
    (2048, 5120, 34816, "DEFAULT", "NK", 3, 0),      # the dx GEMM over K = 2I
])
def test_split_choice(m, n, k, epi, layout, splits, tail0):
    f = fields(ep.describe_plan(m, n, k, epi, BF16, b_layout=layout))
    assert (int(f["splits"]), int(f["split_tail0"])) == (splits, tail0), f


def test_split_choice_transposed_a_and_ragged_k():
    """The dx-shaped GEMM with A given K x M splits like A given M x K; with K not a multiple
    of 64 it runs register-staged configuration 8, still split 3 ways."""
    for a_layout, k, cfg in (("MK", 34816, 11), ("KM", 34816, 11), ("MK", 34808, 8)):
        f = fields(ep.describe_plan(2048, 5120, k, "DEFAULT", F16, b_layout="NK", a_layout=a_layout))
        assert (f["tile_cfg"], f["splits"]) == (str(cfg), "3"), f


@pytest.mark.parametrize("m,n,k,layout,want_cfg", [
    (5120, 17408, 2048, "KN", 12),   # dW_down = dout^T h: two barriers per k-step for K x N B
    (34816, 5120, 2048, "KN", 12),   # [dW_gate; dW_up] = [d_gate | d_up]^T x
    (34816, 5120, 2048, "NK", 11),   # ... with B given N x K: one barrier
    (65536, 8192, 16384, "KN", 11),  # long K over many rounds: one barrier
])
def test_tile_choice_transposed_a(m, n, k, layout, want_cfg):
    """A given K x M (weight gradients) takes the 64-deep configurations by the B layout's
    rule, as A given M x K does."""
    f = fields(ep.describe_plan(m, n, k, "DEFAULT", BF16, b_layout=layout, a_layout="KM"))
    assert (f["tile_cfg"], f["splits"]) == (str(want_cfg), "1"), f


def test_headline_plans():
    """The H200-shape layer step: forward RELU_AUX_BIAS on configuration 11 over 256 x 32
    tiles, unsplit, no workspace; backward DRELU_BGRAD on configuration 11 over 256 x 64 tiles
    with the two-pass bias gradient's per-M-tile partials (256 x 16384 floats) as workspace."""
    f = fields(ep.describe_plan(65536, 8192, 16384, "RELU_AUX_BIAS", F16, b_layout="KN"))
    assert (f["tile_cfg"], f["grid"], f["splits"], f["workspace_bytes"]) == ("11", "256x32", "1", "0"), f
    f = fields(ep.describe_plan(65536, 16384, 8192, "DRELU_BGRAD", F16, b_layout="NK"))
    assert (f["tile_cfg"], f["grid"], f["splits"]) == ("11", "256x64", "1"), f
    assert int(f["workspace_bytes"]) == 256 * 16384 * 4, f
    info = ep.describe_plan(65536, 16384, 8192, "DRELU_BGRAD", F16, b_layout="NK", bgrad_mode="atomic")
    assert fields(info)["workspace_bytes"] == "0" and "atomic bgrad" in info, info
    info = ep.describe_plan(4096, 4096, 4096, "RELU_AUX_BIAS", F16, b_layout="KN", path="unfused")
    assert "path=unfused" in info and info.endswith("+ bias_add + relu_pack"), info


@pytest.mark.parametrize("cus", [64, 128, 200, 256, 304])
def test_split_tail_covers_only_the_last_round(cus):
    """Whatever the CU count, a split of the last round leaves the whole rounds unsplit
    (tail0 = whole rounds x slots) and splits fewer tiles than one round holds."""
    for m, n, k, epi, layout in ((2048, 17408, 5120, "DSWIGLU", "KN"), (2048, 17408, 5120, "SWIGLU", "NK"),
                                 (3000, 9000, 4096, "RELU_AUX_BIAS", "KN"), (1000, 30000, 2048, "DEFAULT", "NK")):
        f = fields(ep.describe_plan(m, n, k, epi, BF16, b_layout=layout, cus=cus))
        tiles = eval(f["grid"].replace("x", "*"))
        slots = cus * (2 if "_2wg" in f["tile"] else 1)
        tail0 = int(f["split_tail0"])
        if tail0:
            assert int(f["splits"]) > 1 and tail0 == tiles // slots * slots and 0 < tiles - tail0 < slots, (cus, f)
        if int(f["splits"]) > 1 and not tail0:
            assert tiles < slots, (cus, f)  # every tile split only when the grid is under one round


def test_explicit_options_are_honoured():
    f = fields(ep.describe_plan(2048, 5120, 4096, "DEFAULT", F16, b_layout="NK", tile_cfg=0, split_k=2))
    assert (f["tile_cfg"], f["splits"]) == ("0", "2"), f
    f = fields(ep.describe_plan(2048, 17408, 5120, "DSWIGLU", BF16, b_layout="KN", split_k=3, split_tail=True))
    assert (f["splits"], f["split_tail0"]) == ("3", "512"), f


def test_refusals():
    with pytest.raises(ep.EPError, match="EP_ERR_INVALID_ARG.*cus"):
        ep.describe_plan(256, 256, 256, cus=0)
    with pytest.raises(ep.EPError, match="EP_ERR_UNSUPPORTED.*256-row B tile"):
        ep.describe_plan(2048, 8192, 4096, "SWIGLU", BF16, b_layout="KN", tile_cfg=1)
    with pytest.raises(ep.EPError, match="EP_ERR_UNSUPPORTED.*multiple of 64"):
        ep.describe_plan(2048, 8192, 4072, "DEFAULT", F16, b_layout="NK", tile_cfg=11)
    with pytest.raises(ep.EPError, match="EP_ERR_UNSUPPORTED.*partly filled last round"):
        ep.describe_plan(16384, 17408, 5120, "DSWIGLU", BF16, b_layout="KN", split_k=2, split_tail=True)
    with pytest.raises(ep.EPError, match="EP_ERR_INVALID_ARG"):
        ep.describe_plan(0, 256, 256)


def test_largest_grids():
    """M = 2^31 - 1 rows plan on 256-row tiles (2^23 workgroups: 2^31 threads); 128-row tiles
    would need 2^32 threads in one launch, more than a launch can count, and are refused, as is
    a grid of 2^31 - 1 by 2^22 - 8 outputs (the widest D a leading dimension below 2^22 allows)."""
    mmax = (1 << 31) - 1
    f = fields(ep.describe_plan(mmax, 8, 8, "RELU_AUX_BIAS", F16, b_layout="KN"))
    assert f["grid"] == "8388608x1" and f["tile"].startswith("256x"), f
    f = fields(ep.describe_plan(mmax, 8, 8, "DRELU_BGRAD", BF16, b_layout="NK"))
    assert int(f["workspace_bytes"]) == 8388608 * 8 * 4, f
    with pytest.raises(ep.EPError, match="EP_ERR_UNSUPPORTED.*exceeds one launch"):
        ep.describe_plan(mmax, 8, 8, "DEFAULT", F16, b_layout="KN", tile_cfg=1)
    with pytest.raises(ep.EPError, match="EP_ERR_UNSUPPORTED.*exceeds one launch"):
        ep.describe_plan(mmax, (1 << 22) - 8, 8, "DEFAULT", F16, b_layout="NK")


def test_longest_k():
    """K up to 2^31 - 64 (A given K x M and B K x N, the one layout pair whose leading
    dimensions do not bound K): one 8 x 8 tile, split into the most ranges."""
    kmax = (1 << 31) - 64
    f = fields(ep.describe_plan(8, 8, kmax, "DEFAULT", F16, b_layout="KN", a_layout="KM"))
    assert (f["grid"], f["splits"]) == ("1x1", "8"), f
    with pytest.raises(ep.EPError, match="EP_ERR_UNSUPPORTED.*k must be"):
        ep.describe_plan(8, 8, kmax + 8, "DEFAULT", F16, b_layout="KN", a_layout="KM")
