#!/usr/bin/env python3
"""Benchmark of the fused GEMM + epilogue library on one MI355X.

Prints ONE JSON line.  The headline workload is the fp16 ReLU linear layer at the H200 shape
of "Fusing Matmul Epilogs with nvmath-python" ("Suitable evaluation scenarios"): X 65536 x 16384,
W 16384 x 8192.  One step is the fused forward RELU_AUX_BIAS (Y and its relu_aux) followed by
the fused backward DRELU_BGRAD (dY W^T masked by a separate 65536 x 16384 relu_aux, plus the
bias gradient).  `value` is that step's GEMM throughput in TFLOP/s (2*M*N*K per GEMM; epilog
flops not counted).  The same line carries the unfused-path step time (same GEMM core,
DEFAULT epilog, separate kernels through HBM) and, under "configs", the execute latency of the
launch-bound 32 x 64 x 128 layer, the square 4096^3 layer,
the bf16 SwiGLU forward (M 2048, H 5120, I 17408), the GEMM + dSwiGLU backward (M 16384), a
whole SwiGLU-MLP training step, an M sweep, the GELU layer, launch overhead and plan-time
tuning.  Where stated, torch (hipBLASLt GEMMs plus elementwise ops) runs the same step as a
vendor-library reference.

Timing: HIP events on the stream the kernels run on.  The layers run their steps back to
back over enough copies of their inputs that together exceed the 256 MB Infinity Cache (one
copy at the H200 shape), so no step finds its operands cached, with one event pair around
each block of steps; fused, unfused and torch blocks alternate, so clock and power drift over
the run reach each alike.  The other workloads time one event pair per step, with a 512 MiB
buffer overwritten between steps (outside the events), the variants alternating step by
step.  An event record costs about 6 us of GPU time before the next launch, so per-kernel
durations (the roofline's average launch) come from launches run back to back between a
single event pair.  Inputs are seeded synthetic tensors generated on the device.  The CPU
oracle (float64 numpy) is timed on this host on a sample of each large workload (seeded
output tiles and bias-gradient columns), and whole for the 32 x 64 x 128 and 4096^3 layers, as a
baseline only.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

PEAK_F16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense fp16/bf16 FLOP/clk/CU


def algo_bytes_fwd(m, n, k):
    """Algorithmic HBM bytes of one RELU_AUX_BIAS forward launch: read X (m x k), W (k x n)
    and the bias once; write Y (m x n) and the relu_aux words (m x ceil(n/32)) once."""
    return 2 * (m * k + k * n + n + m * n) + 4 * m * ((n + 31) // 32)
METRIC = "fused GEMM+epilogue TFLOP/s, % MFMA peak, speedup vs unfused path"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-large", action="store_true", help="skip the large-workload summary")
    ap.add_argument("--only", default=None,
                    help="profile helper: run only one workload's fused path "
                         "(sq4096, h200, swiglu, dswiglu, mlp_step, gelu) and print its line")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--calib-copy", type=int, default=0,
                    help="profile helper: first run one device-to-device copy of this many bytes "
                         "(the known-size reference for HBM byte counters)")
    return ap.parse_args()


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_gemm_relu_aux_bias_f16_KN_65536x8192x16384.txt")


def measured_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summary, or None when it is missing or was measured on different kernel sources."""
    try:
        from dense_gemm_epilogues_amd.profiling import read_record, source_hash
        rec = read_record(path)
        if rec.get("source_hash") != source_hash():
            return None
        return rec
    except Exception:
        return None


class Timer:
    """Per-step HIP event pairs on torch's current stream (the stream ep_execute uses)."""

    def __init__(self, n):
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]

    def ms(self):
        return [a.elapsed_time(b) for a, b in self.ev]


def flush_cache(buf):
    if buf is not None:
        buf.zero_()


def run_interleaved(variants, steps, warmup, flush, per_fn=False):
    """variants: {name: [fns forming one step]}.  The variants' steps alternate (a flushed
    step of each in turn), so that clock and power drift over the run reach every variant
    alike.  Returns {name: (step_ms list, per-fn lists or [])}."""
    names = list(variants)
    for _ in range(warmup):
        for nm in names:
            flush_cache(flush)
            for f in variants[nm]:
                f()
    torch.cuda.synchronize()
    marks = {nm: [[torch.cuda.Event(enable_timing=True) for _ in range((len(variants[nm]) if per_fn else 1) + 1)]
                  for _ in range(steps)] for nm in names}
    for st in range(steps):
        for nm in names:
            flush_cache(flush)
            m = marks[nm][st]
            m[0].record()
            for i, f in enumerate(variants[nm]):
                f()
                if per_fn:
                    m[i + 1].record()
            if not per_fn:
                m[1].record()
    torch.cuda.synchronize()
    out = {}
    for nm in names:
        ms = marks[nm]
        n = len(ms[0]) - 1
        out[nm] = ([m[0].elapsed_time(m[n]) for m in ms],
                   [[m[i].elapsed_time(m[i + 1]) for m in ms] for i in range(n)] if per_fn else [])
    return out


def run_rotating(variants, steps, warmup):
    """variants: {name: [one step's fns for input set 0, for set 1, ...]}.  Exactly `steps`
    steps of each variant are timed, back to back, cycling through its input sets (whose
    total exceeds the Infinity Cache, so every step reads its operands from HBM), in 4 blocks
    of steps/4 with one event pair each (one block if steps is not a multiple of 4); the
    variants' blocks alternate, so that clock drift reaches each alike.  Returns {name:
    per-step ms of each block}."""
    names = list(variants)
    for nm in names:
        for st in range(warmup):
            for f in variants[nm][st % len(variants[nm])]:
                f()
    torch.cuda.synchronize()
    blocks = 4 if steps % 4 == 0 and steps >= 8 else 1
    per = steps // blocks
    ev = {nm: [] for nm in names}
    idx = {nm: 0 for nm in names}
    for _ in range(blocks):
        for nm in names:
            sets = variants[nm]
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(per):
                for f in sets[idx[nm] % len(sets)]:
                    f()
                idx[nm] += 1
            e1.record()
            ev[nm].append((e0, e1))
    torch.cuda.synchronize()
    return {nm: [a.elapsed_time(b) / per for a, b in ev[nm]] for nm in names}


def clock_under_load(fns, seconds=1.5, period_s=0.01):
    """Sustained shader clock and socket power while the step `fns` runs back to back for
    `seconds` (batches of 50 steps, synchronised), sampled with amdsmi every `period_s` from a
    second thread.  None when amdsmi is not available."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception:
        return None
    import threading
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                clks = [c for c in m.get("current_gfxclks", []) if isinstance(c, (int, float))]
                pw = m.get("current_socket_power")
                if clks:
                    samples.append((sum(clks) / len(clks), pw if isinstance(pw, (int, float)) else None))
            except Exception:
                pass
            time.sleep(period_s)
    for f in fns:
        f()
    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    steps = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            for f in fns:
                f()
        torch.cuda.synchronize()
        steps += 50
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    if not samples:
        return None
    clk = [c for c, _ in samples]
    pw = [w for _, w in samples if w is not None]
    return {"gfxclk_mhz_mean": round(float(np.mean(clk)), 1), "gfxclk_mhz_min": round(float(np.min(clk)), 1),
            "gfxclk_mhz_max": round(float(np.max(clk)), 1),
            "socket_power_w_mean": round(float(np.mean(pw)), 1) if pw else None, "samples": len(samples),
            "steps": steps, "how": "amdsmi current_gfxclks (mean over XCDs) and current_socket_power, every "
                                  "10 ms while the fused step runs back to back without cache flushes"}


def launch_avg_ms(fn, reps=20):
    """Average duration of fn's launches run back to back between one event pair (operands
    stay in the caches between launches; the event overhead is spread over reps)."""
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def linear_layer(c, steps, warmup, flush, dev, with_unfused=True, with_clock=False):
    """Fused fwd RELU_AUX_BIAS + bwd DRELU_BGRAD (mask chained from the forward), against the
    unfused path and torch.  Steps run back to back over copies of the inputs that together
    exceed the Infinity Cache (see run_rotating); fwd_ms / bwd_ms are the averages of
    back-to-back launches of each half on one input set."""
    import dense_gemm_epilogues_amd as ep
    import workloads as W
    inp = W.linear_inputs(c, device=dev)
    m, n, k = c.m, c.n, c.k
    separate = c.mask_from == "separate"
    names = ["x", "w", "bias", "dy"] + (["mask_in"] if separate else [])
    set_bytes = sum(inp[nm].numel() * inp[nm].element_size() for nm in names) + m * n * 2 + m * k * 2
    nsets = int(min(8, max(1, -(-(768 << 20) // set_bytes))))
    sets = [inp] + [{nm: inp[nm].clone() for nm in names} for _ in range(nsets - 1)]
    paths = ["fused", "unfused"] if with_unfused else ["fused"]
    plans = {path: [] for path in paths}
    for ins in sets:
        for path in paths:
            pf = ep.Plan(ins["x"], ins["w"], "RELU_AUX_BIAS", {"bias": ins["bias"]}, b_layout="KN", path=path)
            _, aux = pf.execute()
            mb = ins["mask_in"] if separate else aux["relu_aux"]
            pb = ep.Plan(ins["dy"], ins["w"], "DRELU_BGRAD", {"relu_aux": mb}, b_layout="NK", path=path)
            plans[path].append((pf, pb))
    variants = {path: [[pf.execute, pb.execute] for pf, pb in plans[path]] for path in paths}
    if with_unfused:
        # vendor-library reference: hipBLASLt GEMMs + torch elementwise, byte mask instead of
        # bits; the bias gradient sums the masked product, as DRELU_BGRAD does
        def torch_step_of(ins):
            x, w, bias, dy = ins["x"], ins["w"], ins["bias"], ins["dy"]
            if separate:  # the separate backward mask (M x K bits) as bytes, unpacked untimed
                bits = torch.arange(32, device=dev, dtype=torch.int32)
                keep_b = ((ins["mask_in"].unsqueeze(-1) >> bits) & 1).to(torch.bool).reshape(m, k)

            def torch_step():
                yy = torch.addmm(bias, x, w).relu_()
                keep = yy > 0
                g = (dy @ w.t()) * (keep_b if separate else keep)
                g.float().sum(0)  # the bias gradient: column sums of the masked product
            return torch_step
        variants["torch"] = [[torch_step_of(ins)] for ins in sets]
    timed = run_rotating(variants, steps, warmup)
    res = {}
    for path in paths:
        st = timed[path]
        pf, pb = plans[path][0]
        res[path] = {"step_ms": float(np.mean(st)), "step_ms_median": float(np.median(st)),
                     "step_ms_min": float(np.min(st)), "step_ms_max": float(np.max(st)),
                     "fwd_ms": launch_avg_ms(pf.execute), "bwd_ms": launch_avg_ms(pb.execute),
                     "fwd_info": pf.info(), "bwd_info": pb.info(), "input_sets": nsets}
    # last, since 1.5 s of continuous load warms the card
    clock = clock_under_load([plans["fused"][0][0].execute, plans["fused"][0][1].execute]) if with_clock else None
    for path in paths:
        for pf, pb in plans[path]:
            pf.free()
            pb.free()
    if with_unfused:
        res["torch"] = {"step_ms": float(np.mean(timed["torch"])), "step_ms_median": float(np.median(timed["torch"]))}
    x, w, bias, dy = inp["x"], inp["w"], inp["bias"], inp["dy"]
    flop = 2.0 * m * n * k
    out = {"flop_per_gemm": flop, "fused": res["fused"]}
    f = res["fused"]
    f["tflops_step"] = 2 * flop / (f["step_ms"] * 1e-3) / 1e12
    f["tflops_fwd"] = flop / (f["fwd_ms"] * 1e-3) / 1e12
    f["tflops_bwd"] = flop / (f["bwd_ms"] * 1e-3) / 1e12
    if with_unfused:
        u = res["unfused"]
        out["unfused"] = u
        # speedups are ratios of medians (the step's mean gives `value`)
        out["speedup_step"] = u["step_ms_median"] / f["step_ms_median"]
        out["speedup_fwd"] = u["fwd_ms"] / f["fwd_ms"]
        out["speedup_bwd"] = u["bwd_ms"] / f["bwd_ms"]
        out["torch"] = res["torch"]
        out["speedup_vs_torch"] = res["torch"]["step_ms_median"] / f["step_ms_median"]
    out["inputs"] = {"x": x, "w": w, "bias": bias, "dy": dy, "mask_in": inp["mask_in"]}
    out["clock"] = clock
    return out


def gelu_layer(c, steps, warmup, flush, dev):
    """Fused GELU_AUX_BIAS forward + DGELU_BGRAD backward (consuming the forward's saved
    pre-activation) against the unfused GEMM + elementwise sequence, on a linear layer's inputs."""
    import dense_gemm_epilogues_amd as ep
    import workloads as W
    inp = W.linear_inputs(c, device=dev)
    x, w, bias, dy = inp["x"], inp["w"], inp["bias"], inp["dy"]
    plans = {}
    for path in ("fused", "unfused"):
        pf = ep.Plan(x, w, "GELU_AUX_BIAS", {"bias": bias}, b_layout="KN", path=path)
        _, aux = pf.execute()
        pb = ep.Plan(dy, w, "DGELU_BGRAD", {"gelu_aux": aux["gelu_aux"]}, b_layout="NK", path=path)
        plans[path] = (pf, pb)
    timed = run_interleaved({p_: [pf.execute, pb.execute] for p_, (pf, pb) in plans.items()}, steps, warmup, flush)
    res = {}
    for path, (pf, pb) in plans.items():
        res[path] = {"step_ms": float(np.median(timed[path][0])), "fwd_ms": launch_avg_ms(pf.execute),
                     "bwd_ms": launch_avg_ms(pb.execute)}
    # the forward epilogs side by side, same method, alternating (3 rounds, medians): what the
    # exact GELU costs over ReLU, with (GELU_AUX_BIAS also writes the M x N pre-activation) and
    # without a saved output
    fwd = {"RELU_AUX_BIAS": ep.Plan(x, w, "RELU_AUX_BIAS", {"bias": bias}, b_layout="KN"),
           "GELU_AUX_BIAS": plans["fused"][0],
           "RELU_BIAS": ep.Plan(x, w, "RELU_BIAS", {"bias": bias}, b_layout="KN"),
           "GELU_BIAS": ep.Plan(x, w, "GELU_BIAS", {"bias": bias}, b_layout="KN")}
    side = {k: [] for k in fwd}
    for _ in range(3):
        for k, p_ in fwd.items():
            side[k].append(launch_avg_ms(p_.execute))
    side = {k: float(np.median(v)) for k, v in side.items()}
    for k in ("RELU_AUX_BIAS", "RELU_BIAS", "GELU_BIAS"):
        fwd[k].free()
    for pf, pb in plans.values():
        pf.free()
        pb.free()
    flop = 2.0 * c.m * c.n * c.k
    f, u = res["fused"], res["unfused"]
    return {"forward_epilogs_ms": {k: round(v, 5) for k, v in side.items()},
            "gelu_aux_over_relu_aux": round(side["GELU_AUX_BIAS"] / side["RELU_AUX_BIAS"], 4),
            "gelu_over_relu": round(side["GELU_BIAS"] / side["RELU_BIAS"], 4),
            "fused_step_tflops": round(2 * flop / (f["step_ms"] * 1e-3) / 1e12, 1),
            "fwd_pct_peak": round(100 * flop / (f["fwd_ms"] * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 2),
            "bwd_pct_peak": round(100 * flop / (f["bwd_ms"] * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 2),
            "fused_fwd_ms": round(f["fwd_ms"], 5), "fused_bwd_ms": round(f["bwd_ms"], 5),
            "unfused_fwd_ms": round(u["fwd_ms"], 5), "unfused_bwd_ms": round(u["bwd_ms"], 5),
            "speedup_step": round(u["step_ms"] / f["step_ms"], 4)}


def swiglu_fwd(c, steps, warmup, flush, dev):
    import dense_gemm_epilogues_amd as ep
    import workloads as W
    inp = W.swiglu_inputs(c, device=dev)
    x, wg, wu, wd = inp["x"], inp["wg"], inp["wu"], inp["wd"]
    m, h, i = c.m, c.h, c.i
    plans = {}
    hs = {}
    for path in ("fused", "unfused"):
        ps = ep.Plan(x, wg, "SWIGLU", {"b2": wu}, b_layout="NK", path=path)
        hh, _ = ps.execute()
        hs[path] = hh
        pd = ep.Plan(hh, wd, "DEFAULT", b_layout="NK")
        plans[path] = (ps, pd)
    # vendor-library reference: hipBLASLt GEMMs and torch's elementwise ops, bf16 as given
    def torch_step():
        hh = torch.nn.functional.silu(x @ wg.t()) * (x @ wu.t())
        hh @ wd.t()
    variants = {p_: [ps.execute, pd.execute] for p_, (ps, pd) in plans.items()}
    variants["torch"] = [torch_step]
    timed = run_interleaved(variants, steps, warmup, flush)
    res = {}
    for path, (ps, pd) in plans.items():
        res[path] = {"step_ms": float(np.median(timed[path][0])), "swiglu_ms": launch_avg_ms(ps.execute),
                     "down_ms": launch_avg_ms(pd.execute), "swiglu_info": ps.info(), "down_info": pd.info()}
        ps.free()
        pd.free()
    f, u = res["fused"], res["unfused"]
    flop_s, flop_d = 2.0 * 2 * m * h * i, 2.0 * m * h * i
    f["tflops_swiglu"] = flop_s / (f["swiglu_ms"] * 1e-3) / 1e12
    f["tflops_down"] = flop_d / (f["down_ms"] * 1e-3) / 1e12
    f["tflops_step"] = (flop_s + flop_d) / (f["step_ms"] * 1e-3) / 1e12
    torch_ms = float(np.median(timed["torch"][0]))
    return {"fused": f, "unfused": u, "speedup_swiglu": u["swiglu_ms"] / f["swiglu_ms"],
            "speedup_step": u["step_ms"] / f["step_ms"], "torch_step_ms": torch_ms,
            "speedup_vs_torch": torch_ms / f["step_ms"], "inputs": inp, "h": hs["fused"]}


def dswiglu_bwd(c, steps, warmup, flush, dev):
    import dense_gemm_epilogues_amd as ep
    import workloads as W
    inp = W.dswiglu_inputs(c, device=dev)
    plans = {path: ep.Plan(inp["dout"], inp["wd"], "DSWIGLU", {"gate": inp["gate"], "up": inp["up"]},
                           b_layout="KN", path=path) for path in ("fused", "unfused")}
    # vendor-library reference, as autograd would run it: dh = dout Wd with hipBLASLt, then
    # torch's own SiLU backward kernel and elementwise products, bf16 tensors throughout
    dout, wd, gate, up = inp["dout"], inp["wd"], inp["gate"], inp["up"]

    def torch_step():
        dh = dout @ wd
        torch.ops.aten.silu_backward(dh * up, gate)  # d_gate
        dh * torch.nn.functional.silu(gate)           # d_up
    variants = {p_: [p.execute] for p_, p in plans.items()}
    variants["torch"] = [torch_step]
    timed = run_interleaved(variants, steps, warmup, flush)
    res = {}
    for path, p in plans.items():
        res[path] = {"ms": float(np.median(timed[path][0])), "info": p.info()}
        p.free()
    flop = 2.0 * c.m * c.h * c.i
    f, u = res["fused"], res["unfused"]
    f["tflops"] = flop / (f["ms"] * 1e-3) / 1e12
    torch_ms = float(np.median(timed["torch"][0]))
    return {"fused": f, "unfused": u, "speedup": u["ms"] / f["ms"], "torch_ms": torch_ms,
            "speedup_vs_torch": torch_ms / f["ms"], "inputs": inp}


def mlp_training_step(c, steps, warmup, flush, dev):
    """One SwiGLU-MLP training step (forward and all four gradients) with this library:
      forward  h, [g | u] = SWIGLU_AUX(x; Wg, Wu); out = h Wd^T
      backward [d_gate | d_up] = DSWIGLU(dout, Wd; g, u); dx = [d_gate | d_up] [Wg; Wu];
               [dWg; dWu] = [d_gate | d_up]^T x and dWd = dout^T h (transposed-A GEMMs).
    The fused path runs 6 kernels; the unfused path replaces SWIGLU_AUX and DSWIGLU by
    their GEMM + elementwise sequences.  torch (hipBLASLt GEMMs and elementwise ops) runs the
    same step as a vendor-library reference.  The three alternate step by step, each step
    timed with an event after every kernel (about 6 us each, alike for all).  FLOP per step:
    18 M H I."""
    import dense_gemm_epilogues_amd as ep
    import workloads as W
    inp = W.swiglu_inputs(c, device=dev)
    x, wg, wu, wd = inp["x"], inp["wg"], inp["wu"], inp["wd"]
    m, hd, idim = c.m, c.h, c.i
    w_gu = torch.cat([wg, wu], dim=0).contiguous()
    dout = W.randn((m, hd), W.seed_of(c.cfg, 6), 1.0, torch.bfloat16, dev)
    dgu = torch.empty((m, 2 * idim), dtype=torch.bfloat16, device=dev)
    plans = {}
    for path in ("fused", "unfused"):
        ps = ep.Plan(x, w_gu[:idim], "SWIGLU_AUX", {"b2": w_gu[idim:]}, b_layout="NK", path=path)
        h, aux = ps.execute()
        gu = aux["gu"]
        pd = ep.Plan(h, wd, "DEFAULT", b_layout="NK")
        pds = ep.Plan(dout, wd, "DSWIGLU", {"gate": gu[:, :idim], "up": gu[:, idim:]}, b_layout="KN",
                      out=dgu[:, :idim], aux_out={"d_up": dgu[:, idim:]}, path=path)
        pdx = ep.Plan(dgu, w_gu, "DEFAULT", b_layout="KN")
        pwgu = ep.Plan(dgu, x, "DEFAULT", b_layout="KN", a_layout="KM")
        pwd = ep.Plan(dout, h, "DEFAULT", b_layout="KN", a_layout="KM")
        plans[path] = (ps, pd, pds, pdx, pwgu, pwd)
    # vendor-library reference: the same step with torch ops (GEMMs via hipBLASLt)
    wgt, wut, wdt = wg.t(), wu.t(), wd.t()

    def torch_step():
        g = x @ wgt
        u = x @ wut
        hh = torch.nn.functional.silu(g.float()).mul_(u.float()).to(torch.bfloat16)
        hh @ wdt
        dh = (dout @ wd).float()
        gf, uf = g.float(), u.float()
        sg = torch.sigmoid(gf)
        dsilu = sg * (1 + gf * (1 - sg))
        dg = (dh * uf * dsilu).to(torch.bfloat16)
        du = (dh * gf * sg).to(torch.bfloat16)
        dg @ wg + du @ wu
        dg.t() @ x
        du.t() @ x
        dout.t() @ hh
    variants = {path: [p_.execute for p_ in pl] for path, pl in plans.items()}
    variants["torch"] = [torch_step]
    timed = run_interleaved(variants, steps, warmup, flush, per_fn=True)
    res = {}
    for path, pl in plans.items():
        res[path] = {"step_ms": float(np.median(timed[path][0])),
                     "per_ms": [float(np.median(v)) for v in timed[path][1]]}
        for p_ in pl:
            p_.free()
    res["torch"] = {"step_ms": float(np.median(timed["torch"][0]))}
    flop = 18.0 * m * hd * idim
    names = ["swiglu_aux_fwd", "down_gemm", "dswiglu", "dx_gemm_K2I", "dw_gate_up_gemm_AKM", "dw_down_gemm_AKM"]
    f, u = res["fused"], res["unfused"]
    return {"fused_step_ms": round(f["step_ms"], 4), "unfused_step_ms": round(u["step_ms"], 4),
            "torch_step_ms": round(res["torch"]["step_ms"], 4),
            "fused_step_tflops": round(flop / (f["step_ms"] * 1e-3) / 1e12, 1),
            "step_pct_peak": round(100 * flop / (f["step_ms"] * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 2),
            "speedup_vs_unfused": round(u["step_ms"] / f["step_ms"], 4),
            "speedup_vs_torch": round(res["torch"]["step_ms"] / f["step_ms"], 4),
            "fused_kernel_ms": {n: round(v, 4) for n, v in zip(names, f["per_ms"])},
            "unfused_kernel_ms": {n: round(v, 4) for n, v in zip(names, u["per_ms"])}}


def swiglu_m_sweep(steps, warmup, flush, dev, ms=(2048, 4096, 8192, 16384)):
    """Fused SWIGLU (both GEMMs and SiLU*mul in one kernel) against the unfused two GEMMs +
    silu_mul at several token counts M, H 5120, I 17408 (the M range of the
    gemm_swiglu_mlp_fusion.py docstring)."""
    import dense_gemm_epilogues_amd as ep
    import workloads as W
    c = W.SWIGLU[4]
    out = {}
    for m in ms:
        inp = W.swiglu_inputs(c, device=dev, m=m)
        plans = {path: ep.Plan(inp["x"], inp["wg"], "SWIGLU", {"b2": inp["wu"]}, b_layout="NK", path=path)
                 for path in ("fused", "unfused")}
        timed = run_interleaved({p_: [p.execute] for p_, p in plans.items()}, steps, warmup, flush)
        res = {path: float(np.median(timed[path][0])) for path in plans}
        for p in plans.values():
            p.free()
        tf = 4.0 * m * c.h * c.i / (res["fused"] * 1e-3) / 1e12
        out[f"M{m}"] = {"fused_ms": round(res["fused"], 4), "unfused_ms": round(res["unfused"], 4),
                        "fused_tflops": round(tf, 1), "pct_peak": round(100 * tf / PEAK_F16_TFLOPS, 2),
                        "speedup": round(res["unfused"] / res["fused"], 4)}
        del inp
        torch.cuda.empty_cache()
    return out


def autotune_vs_model(steps, warmup, flush, dev):
    """Plan-time tuning (ep_options.autotune) against the shape model's choice, on the square
    forward and on the SwiGLU down projection (160 output tiles on 256 CUs)."""
    import dense_gemm_epilogues_amd as ep
    import workloads as W
    out = {}
    c2 = W.LINEAR[2]
    li = W.linear_inputs(c2, device=dev)
    c4 = W.SWIGLU[4]
    si = W.swiglu_inputs(c4, device=dev)
    h = torch.randn(c4.m, c4.i, device=dev).to(torch.bfloat16)
    cases = {"square_fwd_relu_aux_bias": (li["x"], li["w"], "RELU_AUX_BIAS", {"bias": li["bias"]}, "KN"),
             "swiglu_down_gemm": (h, si["wd"], "DEFAULT", {}, "NK")}
    for name, (a, b, epi, ins, lay) in cases.items():
        plans = {"model": ep.Plan(a, b, epi, ins, b_layout=lay),
                 "tuned": ep.Plan(a, b, epi, ins, b_layout=lay, autotune=True)}
        timed = run_interleaved({k: [p.execute] for k, p in plans.items()}, steps, warmup, flush)
        r = {}
        for k, p in plans.items():
            info = p.info()
            r[k] = {"ms": round(float(np.median(timed[k][0])), 4),
                    "tile": info.split("tile=")[1].split()[0], "splits": int(info.split("splits=")[1].split()[0])}
            p.free()
        out[name] = r
    return out


def execute_overhead(dev):
    """What one ep_execute costs apart from the kernels: the host time to enqueue it, the
    end-to-end latency of a 256^3 fp16 GEMM (launch + kernel, synchronised every call; the
    gemm_swiglu_mlp_fusion.py notes quote about 8 us per 256^3 execute on B200), and the fused
    SwiGLU forward (SWIGLU + down GEMM, M 2048) replayed from a captured HIP graph against
    eager launches."""
    import dense_gemm_epilogues_amd as ep
    import workloads as W
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    a = torch.randn(256, 256, device=dev, generator=g).half()
    b = torch.randn(256, 256, device=dev, generator=g).half()
    p = ep.Plan(a, b, "DEFAULT", b_layout="NK")
    for _ in range(50):
        p.execute()
    torch.cuda.synchronize()
    n = 2000
    t0 = time.perf_counter()
    for _ in range(n):
        p.execute()
    t1 = time.perf_counter()
    torch.cuda.synchronize()
    host_us = (t1 - t0) / n * 1e6
    lat = []
    for _ in range(200):
        t0 = time.perf_counter()
        p.execute()
        torch.cuda.synchronize()
        lat.append(time.perf_counter() - t0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        p.execute()
    e1.record()
    torch.cuda.synchronize()
    gpu_us = e0.elapsed_time(e1) / n * 1e3
    p.free()

    c = W.SWIGLU[4]
    inp = W.swiglu_inputs(c, device=dev)
    ps = ep.Plan(inp["x"], inp["wg"], "SWIGLU", {"b2": inp["wu"]}, b_layout="NK")
    hh, _ = ps.execute()
    pd = ep.Plan(hh, inp["wd"], "DEFAULT", b_layout="NK")
    step = lambda: (ps.execute(), pd.execute())
    step()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()  # warm on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    reps = 50
    times = {}
    for name, fn in (("eager", step), ("graph", graph.replay)):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        times[name] = (time.perf_counter() - t0) / reps * 1e3
    ps.free()
    pd.free()
    return {"host_us_per_execute": round(host_us, 2),
            "gemm_256cubed_us_back_to_back": round(gpu_us, 2),
            "gemm_256cubed_us_synchronised": round(float(np.median(lat)) * 1e6, 2),
            "swiglu_fwd_M2048_eager_ms": round(times["eager"], 4),
            "swiglu_fwd_M2048_graph_ms": round(times["graph"], 4)}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def timed_reps(fn, min_s, max_reps):
    """Mean wall time of fn() over repetitions until min_s seconds have passed (at least one,
    at most max_reps)."""
    reps, tot = 0, 0.0
    while reps == 0 or (tot < min_s and reps < max_reps):
        t0 = time.perf_counter()
        fn()
        tot += time.perf_counter() - t0
        reps += 1
    return tot / reps, reps


def host(t):
    """numpy copy of a device tensor (bf16 as its uint16 bits, int32 mask words as uint32)."""
    import workloads as W
    return W.to_numpy(t)


def oracle_rate(sample_flop, step_flop, sec, reps, what, copy_s):
    rate = sample_flop / sec
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{what}; {sample_flop / 1e9:.1f} GFLOP per pass, {reps} pass(es) of {sec:.2f} s; "
                      f"device-to-host copies ({copy_s:.2f} s) not timed; host has {os.cpu_count()} logical CPUs",
            "sample_gflop": round(sample_flop / 1e9, 2),
            "extrapolated_full_step_s": round(step_flop / rate, 1),
            "extrapolated_note": "extrapolated: the whole step's GEMM FLOP at the sampled rate, not measured"}


def cpu_baseline_linear(inp, c, min_s=10.0):
    """The float64 oracle on a sample of the ReLU layer's step, on the same inputs: 32 seeded
    128 x 128 tiles plus the 4 corners of the forward (RELU_AUX_BIAS: Y and mask words) and of
    the backward (DRELU_BGRAD: masked dY W^T), and 64 seeded bias-gradient columns plus the
    first and last (each a full column sum of the masked product over all rows)."""
    import oracle
    m, n, k = c.m, c.n, c.k
    t0 = time.perf_counter()
    ftiles = oracle.sample_tiles(m, n, count=32, seed=31)
    btiles = oracle.sample_tiles(m, k, count=32, seed=37)
    cols = oracle.sample_columns(k, count=64, seed=41)
    bias = host(inp["bias"])
    fwd = [(host(inp["x"][r0:r1]), host(inp["w"][:, c0:c1]), bias[c0:c1]) for (r0, r1, c0, c1) in ftiles]
    words_all = inp["mask_in"]
    bwd = [(host(inp["dy"][r0:r1]), host(inp["w"][c0:c1]), host(words_all[r0:r1, c0 // 32:(c1 + 31) // 32]))
           for (r0, r1, c0, c1) in btiles]
    cwords = sorted(set(int(cc) // 32 for cc in cols))
    widx = np.array([cwords.index(int(cc) // 32) * 32 + int(cc) % 32 for cc in cols])
    dy_h = host(inp["dy"])
    w_cols = host(inp["w"][torch.as_tensor(cols, device=inp["w"].device)])
    words_cols = host(words_all[:, torch.as_tensor(cwords, device=words_all.device)])
    copy_s = time.perf_counter() - t0
    d = oracle.decode_f16

    def run():
        for xt, wt, bt in fwd:
            oracle.relu_aux_bias(d(xt), d(wt), d(bt), "KN")
        for dyt, wr, wd in bwd:
            oracle.drelu_bgrad(d(dyt), d(wr), "NK", wd)
        acc = np.zeros(len(cols))
        w64 = d(w_cols)
        for r0 in range(0, m, 8192):
            g = oracle.matmul(d(dy_h[r0:r0 + 8192]), w64, "NK")
            bits = oracle.unpack_relu_mask(words_cols[r0:r0 + 8192], 32 * len(cwords))[:, widx]
            acc += np.where(bits, g, 0.0).sum(axis=0)
        return acc

    sec, reps = timed_reps(run, min_s, 5)
    flop = sum(2.0 * (r1 - r0) * (c1 - c0) * k for (r0, r1, c0, c1) in ftiles)
    flop += sum(2.0 * (r1 - r0) * (c1 - c0) * n for (r0, r1, c0, c1) in btiles)
    flop += 2.0 * m * n * len(cols)
    what = (f"{len(ftiles)} forward and {len(btiles)} backward 128x128 output tiles and {len(cols)} full "
            f"bias-gradient columns of the {m}x{k}x{n} fp16 layer step (fp64 oracle)")
    return oracle_rate(flop, 2 * 2.0 * m * n * k, sec, reps, what, copy_s)


def cpu_baseline_swiglu(inp, h_gpu, c, min_s=3.0):
    """The oracle on 32 seeded + 4 corner 128 x 128 tiles of the SwiGLU output h (two GEMMs and
    silu*mul each) and as many tiles of the down projection (on the GPU's h)."""
    import oracle
    m, hd, i = c.m, c.h, c.i
    t0 = time.perf_counter()
    ht = oracle.sample_tiles(m, i, count=32, seed=51)
    ot = oracle.sample_tiles(m, hd, count=32, seed=52)
    hs = [(host(inp["x"][r0:r1]), host(inp["wg"][c0:c1]), host(inp["wu"][c0:c1])) for (r0, r1, c0, c1) in ht]
    ds = [(host(h_gpu[r0:r1]), host(inp["wd"][c0:c1])) for (r0, r1, c0, c1) in ot]
    copy_s = time.perf_counter() - t0
    d = oracle.decode_bf16_bits

    def run():
        for xt, g, u in hs:
            oracle.swiglu(d(xt), d(g), d(u))
        for ht_, wd in ds:
            oracle.matmul(d(ht_), d(wd), "NK")

    sec, reps = timed_reps(run, min_s, 5)
    flop = sum(4.0 * (r1 - r0) * (c1 - c0) * hd for (r0, r1, c0, c1) in ht)
    flop += sum(2.0 * (r1 - r0) * (c1 - c0) * i for (r0, r1, c0, c1) in ot)
    what = f"{len(ht)} tiles of h and {len(ot)} tiles of the down projection (bf16 SwiGLU forward, fp64 oracle)"
    return oracle_rate(flop, 6.0 * m * hd * i, sec, reps, what, copy_s)


def cpu_baseline_dswiglu(inp, c, min_s=3.0):
    """The oracle on 32 seeded + 4 corner 128 x 128 tiles of d_gate and d_up."""
    import oracle
    m, hd, i = c.m, c.h, c.i
    t0 = time.perf_counter()
    tl = oracle.sample_tiles(m, i, count=32, seed=53)
    ts = [(host(inp["dout"][r0:r1]), host(inp["wd"][:, c0:c1]), host(inp["gate"][r0:r1, c0:c1]),
           host(inp["up"][r0:r1, c0:c1])) for (r0, r1, c0, c1) in tl]
    copy_s = time.perf_counter() - t0
    d = oracle.decode_bf16_bits

    def run():
        for dt, wd, g, u in ts:
            oracle.dswiglu(d(dt), d(wd), d(g), d(u))

    sec, reps = timed_reps(run, min_s, 5)
    flop = sum(2.0 * (r1 - r0) * (c1 - c0) * hd for (r0, r1, c0, c1) in tl)
    what = f"{len(tl)} tiles of d_gate and d_up (bf16 GEMM + dSwiGLU, fp64 oracle)"
    return oracle_rate(flop, 2.0 * m * hd * i, sec, reps, what, copy_s)


def cpu_oracle_full_linear(inp, c, min_s=3.0):
    """The whole float64 oracle of a ReLU layer step, timed: RELU_AUX_BIAS forward, then
    DRELU_BGRAD backward on the oracle's own forward mask (square layer) or on the separate
    mask (the 32 x 64 x 128 layer)."""
    import oracle
    t0 = time.perf_counter()
    d = oracle.decode_f16
    x, w, bias, dy = (d(host(inp[nm])) for nm in ("x", "w", "bias", "dy"))
    sep = c.mask_from == "separate"
    words_in = host(inp["mask_in"]) if sep else None
    copy_s = time.perf_counter() - t0

    def run():
        _, words, _ = oracle.relu_aux_bias(x, w, bias, "KN")
        oracle.drelu_bgrad(dy, w, "NK", words_in if sep else words)

    sec, reps = timed_reps(run, min_s, 50)
    flop = 2 * 2.0 * c.m * c.n * c.k
    return {"value": flop / sec / 1e12, "unit": "TFLOP/s", "seconds_per_step": sec, "cores": int(blas_threads()),
            "kind": "oracle",
            "sample": f"the whole {c.m}x{c.n}x{c.k} fp16 layer step (forward + backward, fp64 oracle), "
                      f"{reps} pass(es); device-to-host copies ({copy_s:.2f} s) not timed; host has "
                      f"{os.cpu_count()} logical CPUs"}


def tiny_layer(dev, reps=20, warmup=5):
    """The 32 x 64 x 128 fp16 layer (launch-bound; TFLOP/s means nothing there): the latency of
    one execute of the fused RELU_BIAS and RELU_AUX_BIAS forwards and of the DRELU_BGRAD
    backward (its GEMM launch plus the bias-gradient pass), one HIP event pair per execute on
    the launch stream, after warm-up executes; median, min and max over the timed ones."""
    import dense_gemm_epilogues_amd as ep
    import workloads as W
    c = W.LINEAR[1]
    inp = W.linear_inputs(c, device=dev)
    plans = {"fwd_relu_bias": ep.Plan(inp["x"], inp["w"], "RELU_BIAS", {"bias": inp["bias"]}, b_layout="KN"),
             "fwd_relu_aux_bias": ep.Plan(inp["x"], inp["w"], "RELU_AUX_BIAS", {"bias": inp["bias"]},
                                          b_layout="KN"),
             "bwd_drelu_bgrad": ep.Plan(inp["dy"], inp["w"], "DRELU_BGRAD", {"relu_aux": inp["mask_in"]},
                                        b_layout="NK")}
    out = {"m": c.m, "n": c.n, "k": c.k, "timing": f"{warmup} warm-up, {reps} timed executes, one event pair each"}
    for name, p in plans.items():
        for _ in range(warmup):
            p.execute()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            p.execute()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        out[f"{name}_us"] = {"median": round(float(np.median(ts)), 2), "min": round(float(np.min(ts)), 2),
                             "max": round(float(np.max(ts)), 2)}
        out[f"{name}_kernels"] = p.info().split("kernels=")[1]
        p.free()
    out["inputs"] = inp
    return out


def linear_summary(r, c):
    f = r["fused"]
    flop = r["flop_per_gemm"]
    return {"fused_step_tflops": round(f["tflops_step"], 1),
            "step_pct_peak": round(100 * f["tflops_step"] / PEAK_F16_TFLOPS, 2),
            "fused_step_ms": round(f["step_ms"], 4), "unfused_step_ms": round(r["unfused"]["step_ms"], 4),
            "speedup_step": round(r["speedup_step"], 4),
            "fused_fwd_tflops": round(f["tflops_fwd"], 1), "fused_bwd_tflops": round(f["tflops_bwd"], 1),
            "fwd_pct_peak": round(100 * f["tflops_fwd"] / PEAK_F16_TFLOPS, 2),
            "bwd_pct_peak": round(100 * f["tflops_bwd"] / PEAK_F16_TFLOPS, 2),
            "fused_fwd_ms": round(f["fwd_ms"], 5), "fused_bwd_ms": round(f["bwd_ms"], 5),
            "unfused_fwd_ms": round(r["unfused"]["fwd_ms"], 5), "unfused_bwd_ms": round(r["unfused"]["bwd_ms"], 5),
            "speedup_fwd": round(r["speedup_fwd"], 4), "speedup_bwd": round(r["speedup_bwd"], 4),
            "torch_step_ms": round(r["torch"]["step_ms"], 4), "speedup_vs_torch": round(r["speedup_vs_torch"], 4),
            "gemm_flop": flop, "input_sets": f["input_sets"]}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the fused GEMM kernels run on one "
                                   "device and no multi-GPU path is implemented", "n_gpus": args.gpus}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU available"}))
        sys.exit(1)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import workloads as W
    import dense_gemm_epilogues_amd as ep
    ep.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    flush = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    if args.calib_copy:
        src = torch.empty(args.calib_copy, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only:
        st, wu = args.steps, args.warmup
        if args.only == "sq4096":
            r = linear_layer(W.LINEAR[2], st, wu, flush, dev, with_unfused=False)
            r.pop("inputs")
        elif args.only == "h200":
            r = linear_layer(W.LINEAR[3], st, wu, flush, dev, with_unfused=False)
            r.pop("inputs")
        elif args.only == "swiglu":
            r = swiglu_fwd(W.SWIGLU[4], st, wu, flush, dev)
            r.pop("h")
            r.pop("inputs")
        elif args.only == "gelu":
            r = gelu_layer(W.LINEAR[2], st, wu, flush, dev)
        elif args.only == "mlp_step":
            r = mlp_training_step(W.SWIGLU[4], st, wu, flush, dev)
        elif args.only == "dswiglu":
            r = dswiglu_bwd(W.SWIGLU[5], st, wu, flush, dev)
            r.pop("inputs")
        else:
            raise SystemExit(f"unknown --only {args.only}")
        print(json.dumps({"only": args.only, "result": r}, default=str))
        return

    c3 = W.LINEAR[3]
    t_start = time.time()
    r3 = linear_layer(c3, args.steps, args.warmup, flush, dev, with_clock=True)
    f3 = r3["fused"]
    fwd_tflops = f3["tflops_fwd"]
    line = {
        "metric": METRIC,
        "value": round(f3["tflops_step"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(f3["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "H200-shape ReLU linear layer, fp16 in / fp32 acc: fused RELU_AUX_BIAS forward "
                               "(X 65536x16384 . W 16384x8192 + bias, Y 65536x8192 and its relu_aux) then fused "
                               "DRELU_BGRAD backward (dY 65536x8192 . W^T masked by a separate 65536x16384 "
                               "relu_aux, + bgrad of length 16384)",
                   "m": c3.m, "n": c3.n, "k": c3.k,
                   "cache": "cold: the step's operands (6.5 GB) exceed the 256 MB Infinity Cache"},
        "timing": "4 blocks of steps/4 back-to-back steps per variant, one HIP event pair per block, "
                  "fused / unfused / torch blocks alternating; ms_per_step and value are the mean over the "
                  "blocks, median/min/max are over the blocks, speedups are ratios of the medians",
        "ms_per_step_median": round(f3["step_ms_median"], 4),
        "ms_per_step_min": round(f3["step_ms_min"], 4), "ms_per_step_max": round(f3["step_ms_max"], 4),
        "pct_peak": round(100.0 * f3["tflops_step"] / PEAK_F16_TFLOPS, 2),
        "speedup_vs_unfused": round(r3["speedup_step"], 4),
        "unfused_ms_per_step": round(r3["unfused"]["step_ms"], 4),
        "torch_ms_per_step": round(r3["torch"]["step_ms"], 4),
        "speedup_vs_torch": round(r3["speedup_vs_torch"], 4),
        "fwd_ms": round(f3["fwd_ms"], 4), "bwd_ms": round(f3["bwd_ms"], 4),
        "fwd_tflops": round(f3["tflops_fwd"], 1), "bwd_tflops": round(f3["tflops_bwd"], 1),
        "speedup_fwd_vs_unfused": round(r3["speedup_fwd"], 4), "speedup_bwd_vs_unfused": round(r3["speedup_bwd"], 4),
        "roofline": {"bound": "mfma", "kernel": f3["fwd_info"].split("kernels=")[1],
                     "achieved": round(fwd_tflops, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fwd_tflops / PEAK_F16_TFLOPS, 4), "traffic": None,
                     "algorithmic_per_launch": f"{r3['flop_per_gemm']:.6g} FLOP (2*65536*8192*16384)",
                     "algorithmic_bytes_per_launch": algo_bytes_fwd(c3.m, c3.n, c3.k),
                     "avg_launch_ms": round(f3["fwd_ms"], 4),
                     "avg_launch_how": "20 back-to-back launches of the forward between one HIP event pair "
                                       "on the launch stream"},
        "bwd_kernel": f3["bwd_info"].split("kernels=")[1],
    }
    line["clock_under_load"] = r3["clock"]
    tr = measured_traffic()
    if tr is not None:
        line["roofline"]["traffic"] = round(tr["traffic_bytes_per_launch"])
        line["roofline"]["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    cpu = {}
    if not args.no_cpu:
        cpu["h200"] = cpu_baseline_linear(r3["inputs"], c3)
    r3.pop("inputs")
    torch.cuda.empty_cache()
    if not args.no_large:
        large = {}
        r1 = tiny_layer(dev)
        if not args.no_cpu:
            r1["cpu_oracle_full"] = cpu_oracle_full_linear(r1["inputs"], W.LINEAR[1], min_s=0.5)
        r1.pop("inputs")
        large["tiny_fp16_32x64x128"] = r1
        r2 = linear_layer(W.LINEAR[2], args.steps, args.warmup, flush, dev)
        large["square_fp16_4096x4096x4096"] = linear_summary(r2, W.LINEAR[2])
        if not args.no_cpu:
            large["square_fp16_4096x4096x4096"]["cpu_oracle_full"] = cpu_oracle_full_linear(r2["inputs"], W.LINEAR[2])
        r2.pop("inputs")
        tr2 = measured_traffic(os.path.join(PROFILES, "traffic_gemm_relu_aux_bias_f16_KN_4096.txt"))
        large["square_fp16_4096x4096x4096"]["fwd_traffic_bytes"] = (round(tr2["traffic_bytes_per_launch"])
                                                                    if tr2 is not None else None)
        torch.cuda.empty_cache()
        s_l, w_l = max(3, args.steps // 4), max(1, args.warmup // 2)
        r4 = swiglu_fwd(W.SWIGLU[4], args.steps, args.warmup, flush, dev)
        large["swiglu_fwd_bf16_M2048_H5120_I17408"] = {
            "fused_swiglu_tflops": round(r4["fused"]["tflops_swiglu"], 1),
            "swiglu_pct_peak": round(100 * r4["fused"]["tflops_swiglu"] / PEAK_F16_TFLOPS, 2),
            "down_gemm_tflops": round(r4["fused"]["tflops_down"], 1),
            "fused_swiglu_ms": round(r4["fused"]["swiglu_ms"], 4),
            "unfused_swiglu_ms": round(r4["unfused"]["swiglu_ms"], 4),
            "speedup_swiglu": round(r4["speedup_swiglu"], 4), "speedup_fwd_step": round(r4["speedup_step"], 4),
            "torch_fwd_step_ms": round(r4["torch_step_ms"], 4), "speedup_fwd_step_vs_torch": round(r4["speedup_vs_torch"], 4)}
        if not args.no_cpu:
            large["swiglu_fwd_bf16_M2048_H5120_I17408"]["cpu_oracle_sampled"] = cpu_baseline_swiglu(
                r4["inputs"], r4["h"], W.SWIGLU[4])
        del r4
        torch.cuda.empty_cache()
        r5 = dswiglu_bwd(W.SWIGLU[5], args.steps, args.warmup, flush, dev)
        large["dswiglu_bwd_bf16_M16384_H5120_I17408"] = {
            "fused_tflops": round(r5["fused"]["tflops"], 1),
            "pct_peak": round(100 * r5["fused"]["tflops"] / PEAK_F16_TFLOPS, 2),
            "fused_ms": round(r5["fused"]["ms"], 4), "unfused_ms": round(r5["unfused"]["ms"], 4),
            "speedup": round(r5["speedup"], 4), "torch_ms": round(r5["torch_ms"], 4),
            "speedup_vs_torch": round(r5["speedup_vs_torch"], 4)}
        if not args.no_cpu:
            large["dswiglu_bwd_bf16_M16384_H5120_I17408"]["cpu_oracle_sampled"] = cpu_baseline_dswiglu(
                r5["inputs"], W.SWIGLU[5])
        del r5
        torch.cuda.empty_cache()
        large["swiglu_fwd_bf16_M_sweep_H5120_I17408"] = swiglu_m_sweep(s_l, w_l, flush, dev)
        large["swiglu_mlp_training_step_bf16_M2048_H5120_I17408"] = mlp_training_step(W.SWIGLU[4], args.steps, args.warmup, flush, dev)
        torch.cuda.empty_cache()
        large["gelu_layer_fp16_4096x4096x4096"] = gelu_layer(W.LINEAR[2], args.steps, args.warmup, flush, dev)
        large["execute_overhead"] = execute_overhead(dev)
        large["autotune_vs_model"] = autotune_vs_model(s_l, w_l, flush, dev)
        line["configs"] = large
    if not args.no_cpu:
        line["cpu_baseline"] = cpu["h200"]
    line["wall_s"] = round(time.time() - t_start, 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
