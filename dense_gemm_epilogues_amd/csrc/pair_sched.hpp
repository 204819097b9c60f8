// Load schedule of the k-step pairs of the 16x16 GEMM kernels: plain C++ (no device code),
// so that host programs can check it.
#pragma once

namespace ep {

// Load schedule of the k-step pairs (in gemm_kernel).  Of a wave's N_DMA load slots per
// stage, nps are paired: the 2 nps loads of the pair (k-steps kt+3, kt+4; kt odd) run one
// every ps MFMAs from the odd k-step's barrier (MFMA hb) on, pafter of them in that k-step and
// the rest before the next k-step's barrier.  The other nu slots are loaded every k-step for
// k-step kt+3, one every us MFMAs from MFMA uoff (positions never shared with a paired load).
// vmc_odd / vmc_even: loads younger than the last one of the stage needed next, at the
// barrier of an odd / even k-step; vmc_pro: younger than stage 0's after the prologue.
struct PairSched {
  int ps, pafter, us, uoff, vmc_odd, vmc_even, vmc_pro;
};
constexpr PairSched pair_sched(int nmma, int hb, int nps, int nu, int n_dma) {
  PairSched s{};
  s.ps = nmma / (2 * nps);
  s.pafter = (nmma - hb) / s.ps;
  s.us = nu > 0 ? nmma / nu : nmma;
  s.uoff = s.ps / 2;
  // position of paired load d (in its k-step) and whether it is issued in the odd k-step
  auto ppos = [&](int d) { return d < s.pafter ? hb + s.ps * d : (d - s.pafter) * s.ps; };
  // loads of a k-step of parity par at MFMA positions > pos (par 0 even, 1 odd)
  auto after = [&](int par, int pos) {
    int n = 0;
    for (int d = 0; d < 2 * nps; ++d)
      if ((d < s.pafter) == (par == 1) && ppos(d) > pos) ++n;
    for (int j = 0; j < nu; ++j)
      if (s.uoff + s.us * j > pos) ++n;
    return n;
  };
  auto before_barrier = [&](int par) {
    int n = 0;
    for (int d = 0; d < 2 * nps; ++d)
      if ((d < s.pafter) == (par == 1) && ppos(d) < hb) ++n;
    for (int j = 0; j < nu; ++j)
      if (s.uoff + s.us * j < hb) ++n;
    return n;
  };
  // odd kt needs k-step kt+1: unpaired loads from k-step kt-2, paired loads as the first of
  // the pair begun in kt-2, the last of which (the last even d) is issued in k-step kt-1
  int last3 = 0;
  for (int d = s.pafter; d < 2 * nps; ++d)
    if (d % 2 == 0) last3 = ppos(d);
  s.vmc_odd = after(0, last3) + before_barrier(1);
  // even kt needs k-step kt+1: its unpaired loads and the pair's second half both come last
  // in k-step kt-2; then all of k-step kt-1 and what kt issues before its barrier
  int lastl = ppos(2 * nps - 1);
  if (nu > 0 && s.uoff + s.us * (nu - 1) > lastl) lastl = s.uoff + s.us * (nu - 1);
  s.vmc_even = after(0, lastl) + after(1, -1) + before_barrier(0);
  // prologue: k-steps 0 and 1, the unpaired loads of k-step 2, the pair (2, 3)'s first pafter
  s.vmc_pro = n_dma + nu + s.pafter;
  return s;
}

}  // namespace ep
