"""Host check of the k-step pair load schedule of the 16x16 GEMM kernels (no GPU).

The kernels wait at each k-step's barrier with `s_waitcnt vmcnt(N)`: every load older than
the N youngest must have landed.  `pair_sched` (csrc/pair_sched.hpp) derives N from the load
positions.  Here a host build of that header reports its numbers, and an independent
simulation of the issue order over many k-steps checks that, at every barrier, each load of
the stage needed next is older than the N youngest, that every (k-step, slot) is loaded
exactly once, and that no load targets a stage before the barrier that frees it.

The simulated order follows the kernel's placement rules (a 4-stage ring, one MFMA index g
per position in a k-step, the barrier at MFMA hb):
  - prologue: k-steps 0 and 1 (all slots), k-step 2's unpaired slots, then the first pafter
    loads of the pair (2, 3);
  - odd k-step kt, g >= hb, (g - hb) % ps == 0: pair load d = (g - hb) / ps, slot d / 2 of
    k-step kt + 3 + d % 2;
  - even k-step kt, g < hb, g % ps == 0: pair load d = pafter + g / ps, slot d / 2 of
    k-step kt + 2 + d % 2;
  - every k-step, g % us == uoff: unpaired slot nps + g / us of k-step kt + 3.
Stage L % 4 is free once k-step L - 4's barrier has passed (its fragments were read in
k-step L - 5 and waited for before that barrier).
"""
import os
import re
import shutil
import subprocess
from collections import Counter

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_gemm_epilogues_amd", "csrc")

# (nmma, hb, nps, nu, n_dma): the kernels' two uses (256x256 tiles, 4 waves, 64 MFMAs per
# k-step, barrier after 16; N x K B pairs all 8 slots, K x N B pairs A's 4) and one more split
CASES = [(64, 16, 8, 0, 8), (64, 16, 4, 4, 8), (64, 16, 4, 2, 6)]

PROGRAM = r"""
#include <cstdio>
#include "pair_sched.hpp"
int main() {
  const int c[][5] = {%s};
  for (const auto& x : c) {
    const ep::PairSched s = ep::pair_sched(x[0], x[1], x[2], x[3], x[4]);
    std::printf("%%d %%d %%d %%d %%d %%d %%d\n", s.ps, s.pafter, s.us, s.uoff, s.vmc_odd, s.vmc_even, s.vmc_pro);
  }
}
"""


@pytest.fixture(scope="module")
def schedules(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("pair_sched")
    src = d / "ps.cpp"
    src.write_text(PROGRAM % ", ".join("{%d, %d, %d, %d, %d}" % c for c in CASES))
    exe = d / "ps"
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    return {c: tuple(int(v) for v in line.split()) for c, line in zip(CASES, out)}


def simulate(nmma, hb, nps, nu, n_dma, sched, ksteps=40):
    ps, pafter, us, uoff, vmc_odd, vmc_even, vmc_pro = sched
    nslots = nps + nu
    assert nslots == n_dma
    ops = []    # (k-step loaded, slot) in issue order
    when = {}   # (k-step, slot) -> issue time (k-step * nmma + g); prologue at -1
    def issue(op, t):
        ops.append(op)
        when.setdefault(op, []).append(t)
    for L in (0, 1):
        for s in range(nslots):
            issue((L, s), -1)
    for j in range(nu):
        issue((2, nps + j), -1)
    for d in range(pafter):
        issue((2 + d % 2, d // 2), -1)
    # after the prologue the kernel waits for stage 0
    assert vmc_pro <= len(ops)
    assert all(op[0] != 0 for op in ops[len(ops) - vmc_pro:])
    assert all((0, s) in ops[:len(ops) - vmc_pro] for s in range(nslots))
    for kt in range(ksteps):
        odd = kt % 2 == 1
        for g in range(nmma):
            if g == hb:
                v = vmc_odd if odd else vmc_even
                older = set(ops[:len(ops) - v])
                for s in range(nslots):
                    assert (kt + 1, s) in older, (kt, s, v)
            t = kt * nmma + g
            if odd and g >= hb and (g - hb) % ps == 0:
                d = (g - hb) // ps
                issue((kt + 3 + d % 2, d // 2), t)
            elif not odd and g < hb and g % ps == 0:
                d = pafter + g // ps
                issue((kt + 2 + d % 2, d // 2), t)
            if nu and g % us == uoff:
                issue((kt + 3, nps + g // us), t)
    count = Counter(ops)
    assert max(count.values()) == 1, [op for op, n in count.items() if n > 1][:4]
    for L in range(ksteps):
        for s in range(nslots):
            assert (L, s) in count, (L, s)
    for (L, s), ts in when.items():
        if L >= 4:
            assert ts[0] >= (L - 4) * nmma + hb, ("stage not yet free", L, s, ts[0])
    return ops


@pytest.mark.parametrize("case", CASES)
def test_pair_schedule_waits(schedules, case):
    nmma, hb, nps, nu, n_dma = case
    ps, pafter, us, uoff, vmc_odd, vmc_even, vmc_pro = schedules[case]
    # placement invariants the kernel asserts at compile time
    assert ps >= 2 and hb % ps == 0 and (nmma - hb) % ps == 0 and pafter < 2 * nps
    assert nu == 0 or (nmma % nu == 0 and us % ps == 0 and uoff % ps != 0)
    assert max(vmc_odd, vmc_even, vmc_pro) <= 63
    simulate(nmma, hb, nps, nu, n_dma, schedules[case])


def test_pair_schedule_waits_are_tight(schedules):
    """One load fewer in flight at either barrier would make it wait for a younger stage
    (the counts are exact, not merely safe): with N+1 the needed stage is not covered."""
    for case in CASES[:2]:
        nmma, hb, nps, nu, n_dma = case
        ps, pafter, us, uoff, vmc_odd, vmc_even, vmc_pro = schedules[case]
        for loose in ((vmc_odd + 1, vmc_even), (vmc_odd, vmc_even + 1)):
            with pytest.raises(AssertionError):
                simulate(nmma, hb, nps, nu, n_dma, (ps, pafter, us, uoff) + loose + (vmc_pro,))


def test_kernel_uses_pair_sched():
    """The kernel takes its barrier and prologue waits from pair_sched."""
    src = open(os.path.join(CSRC, "gemm_kernel.hpp")).read()
    assert re.search(r"PS_\.vmc_even\s*:\s*PS_\.vmc_odd", src)
    assert "PS_.vmc_pro" in src
