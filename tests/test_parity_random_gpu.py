"""Seeded random sweep of the parity check: random ragged shapes (m 1..700, n and k multiples of 8
up to 640) x every epilog x both dtypes x both B layouts x the planner's or an explicit tile
configuration x an optional split-K, each checked against the oracle by the same checker as
the systematic parity tests (run_and_check: tolerances, padding sentinels, mask words, bias
gradients).  A combination the library does not support must be refused with
EP_ERR_UNSUPPORTED for the one documented reason (a dual-B SwiGLU with a K x N weight needs a
256-row B tile); any other refusal fails the test."""
import random

import pytest

from tests import test_parity_small_gpu as T
from tests._gpu import require_gpu, say

pytestmark = pytest.mark.gpu

EPIS = ["DEFAULT", "BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "DRELU_BGRAD", "SWIGLU", "DSWIGLU",
        "GELU_BIAS", "GELU_AUX_BIAS", "DGELU_BGRAD", "SWIGLU_AUX"]


def cases(seed, count):
    rng = random.Random(seed)
    for _ in range(count):
        epi = rng.choice(EPIS)
        dt = rng.choice(["f16", "bf16"])
        lay = rng.choice(["KN", "NK"])
        m = rng.randint(1, 700)
        n = 8 * rng.randint(1, 80)
        k = 8 * rng.randint(1, 80)
        cfg = rng.choice([-1, -1, -1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12])
        split = rng.choice([0, 0, 0, 2, 3, 4])
        if cfg in T.K64_ONLY_CFGS and k % 64:
            k = -(-k // 64) * 64  # (the ragged-K refusal of these has its own test)
        yield epi, dt, lay, m, n, k, cfg, split, rng.randint(0, 10 ** 6)


@pytest.mark.parametrize("seed", [20261203, 7])
def test_random_parity_sweep(seed):
    require_gpu()
    import dense_gemm_epilogues_amd as ep
    refused = 0
    for epi, dt, lay, m, n, k, cfg, split, s in cases(seed, 120):
        say(f"sweep case {epi} {dt} {lay} m={m} n={n} k={k} cfg={cfg} split={split} seed={s}")
        try:
            T.run_and_check(epi, dt, lay, m, n, k, cfg, seed=s, split_k=split)
        except ep.EPError as e:
            msg = str(e)
            assert ("EP_ERR_UNSUPPORTED" in msg and epi in ("SWIGLU", "SWIGLU_AUX") and lay == "KN"
                    and "needs a 256-row B tile" in msg), msg
            refused += 1
    assert refused < 40
