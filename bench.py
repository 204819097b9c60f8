#!/usr/bin/env python3
"""Benchmark of the fused GEMM + epilogue library on one MI355X.

Prints ONE JSON line.  The headline workload is the square fp16 ReLU linear layer
(M = N = K = 4096): one step is the fused forward RELU_AUX_BIAS followed by the fused
backward DRELU_BGRAD that consumes the forward's relu_aux.  `value` is that step's
GEMM throughput in TFLOP/s (2*M*N*K per GEMM; epilog flops not counted).  The same line
carries the unfused-path step time (same GEMM core, DEFAULT epilog, separate kernels
through HBM) and, under "configs", the fused/unfused timings of the large workloads:
the H200-shape fp16 layer (65536 x 16384 x 8192), the bf16 SwiGLU forward
(M 2048, H 5120, I 17408), the GEMM + dSwiGLU backward (M 16384), a whole SwiGLU-MLP
training step, an M sweep, the GELU layer, launch overhead and plan-time tuning.  Where
stated, torch (hipBLASLt GEMMs plus elementwise ops) runs the same step as a vendor-library
reference.

Timing: HIP events on the stream the kernels run on.  The headline layer runs its steps back
to back over several copies of its inputs that together exceed the 256 MB Infinity Cache, so
no step finds its operands cached, with one event pair around each block of steps; fused,
unfused and torch blocks alternate, so clock and power drift over the run reach each alike.
The other workloads time one event pair per step, with a 512 MiB buffer overwritten between
steps (outside the events), the variants alternating step by step.  An event record costs
about 6 us of GPU time before the next launch, so per-kernel durations (the roofline's
average launch) come from launches run back to back between a single event pair.  Inputs are
seeded synthetic tensors generated on the device.  The CPU oracle (float64 numpy) is timed on this host as a baseline only.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

PEAK_F16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense fp16/bf16 FLOP/clk/CU
# read X, W, bias once; write Y and the relu_aux words once (4096^3 fp16 forward)
ALGO_BYTES_SQ4096_FWD = 3 * 4096 * 4096 * 2 + 4096 * 2 + 4096 * 128 * 4
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


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "traffic_gemm_relu_aux_bias_f16_KN_4096.txt")


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summary, or None when it is missing or was measured on different kernel sources."""
    try:
        from dense_gemm_epilogues_amd.profiling import read_record, source_hash
        rec = read_record(TRAFFIC_FILE)
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
        # vendor-library reference: hipBLASLt GEMMs + torch elementwise, byte mask instead of bits
        def torch_step_of(ins):
            x, w, bias, dy = ins["x"], ins["w"], ins["bias"], ins["dy"]
            if separate:  # the separate backward mask (M x K bits) as bytes, unpacked untimed
                bits = torch.arange(32, device=dev, dtype=torch.int32)
                keep_b = ((ins["mask_in"].unsqueeze(-1) >> bits) & 1).to(torch.bool).reshape(m, k)

            def torch_step():
                yy = torch.addmm(bias, x, w).relu_()
                keep = yy > 0
                (dy @ w.t()) * (keep_b if separate else keep)
                dy.float().sum(0)
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
        res["torch"] = {"step_ms": float(np.mean(timed["torch"]))}
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
        out["speedup_step"] = u["step_ms"] / f["step_ms"]
        out["speedup_fwd"] = u["fwd_ms"] / f["fwd_ms"]
        out["speedup_bwd"] = u["bwd_ms"] / f["bwd_ms"]
        out["torch"] = res["torch"]
        out["speedup_vs_torch"] = res["torch"]["step_ms"] / f["step_ms"]
    out["inputs"] = {"x": x, "w": w, "bias": bias, "dy": dy}
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
        res[path] = {"step_ms": float(np.mean(timed[path][0])), "fwd_ms": launch_avg_ms(pf.execute),
                     "bwd_ms": launch_avg_ms(pb.execute)}
        pf.free()
        pb.free()
    flop = 2.0 * c.m * c.n * c.k
    f, u = res["fused"], res["unfused"]
    return {"fused_step_tflops": round(2 * flop / (f["step_ms"] * 1e-3) / 1e12, 1),
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
    for path in ("fused", "unfused"):
        ps = ep.Plan(x, wg, "SWIGLU", {"b2": wu}, b_layout="NK", path=path)
        hh, _ = ps.execute()
        pd = ep.Plan(hh, wd, "DEFAULT", b_layout="NK")
        plans[path] = (ps, pd)
    timed = run_interleaved({p_: [ps.execute, pd.execute] for p_, (ps, pd) in plans.items()}, steps, warmup, flush)
    res = {}
    for path, (ps, pd) in plans.items():
        res[path] = {"step_ms": float(np.mean(timed[path][0])), "swiglu_ms": launch_avg_ms(ps.execute),
                     "down_ms": launch_avg_ms(pd.execute), "swiglu_info": ps.info(), "down_info": pd.info()}
        ps.free()
        pd.free()
    f, u = res["fused"], res["unfused"]
    flop_s, flop_d = 2.0 * 2 * m * h * i, 2.0 * m * h * i
    f["tflops_swiglu"] = flop_s / (f["swiglu_ms"] * 1e-3) / 1e12
    f["tflops_down"] = flop_d / (f["down_ms"] * 1e-3) / 1e12
    f["tflops_step"] = (flop_s + flop_d) / (f["step_ms"] * 1e-3) / 1e12
    return {"fused": f, "unfused": u, "speedup_swiglu": u["swiglu_ms"] / f["swiglu_ms"],
            "speedup_step": u["step_ms"] / f["step_ms"]}


def dswiglu_bwd(c, steps, warmup, flush, dev):
    import dense_gemm_epilogues_amd as ep
    import workloads as W
    inp = W.dswiglu_inputs(c, device=dev)
    plans = {path: ep.Plan(inp["dout"], inp["wd"], "DSWIGLU", {"gate": inp["gate"], "up": inp["up"]},
                           b_layout="KN", path=path) for path in ("fused", "unfused")}
    timed = run_interleaved({p_: [p.execute] for p_, p in plans.items()}, steps, warmup, flush)
    res = {}
    for path, p in plans.items():
        res[path] = {"ms": float(np.mean(timed[path][0])), "info": p.info()}
        p.free()
    flop = 2.0 * c.m * c.h * c.i
    f, u = res["fused"], res["unfused"]
    f["tflops"] = flop / (f["ms"] * 1e-3) / 1e12
    return {"fused": f, "unfused": u, "speedup": u["ms"] / f["ms"]}


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
        res[path] = {"step_ms": float(np.mean(timed[path][0])),
                     "per_ms": [float(np.mean(v)) for v in timed[path][1]]}
        for p_ in pl:
            p_.free()
    res["torch"] = {"step_ms": float(np.mean(timed["torch"][0]))}
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
        res = {path: float(np.mean(timed[path][0])) for path in plans}
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
            r[k] = {"ms": round(float(np.mean(timed[k][0])), 4),
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


def cpu_baseline(inputs, c):
    """The float64 oracle on the same inputs: one full forward + backward step of the square
    layer, repeated until about 10 s of CPU work (at least once)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    x = oracle.decode_f16(inputs["x"].cpu().numpy())
    w = oracle.decode_f16(inputs["w"].cpu().numpy())
    b = oracle.decode_f16(inputs["bias"].cpu().numpy())
    dy = oracle.decode_f16(inputs["dy"].cpu().numpy())
    reps, t_total = 0, 0.0
    while reps == 0 or (t_total < 10.0 and reps < 5):
        t0 = time.perf_counter()
        _, words, _ = oracle.relu_aux_bias(x, w, b, "KN")
        oracle.drelu_bgrad(dy, w, "NK", words)
        t_total += time.perf_counter() - t0
        reps += 1
    flop = 2 * 2.0 * c.m * c.n * c.k
    sec = t_total / reps
    return {"value": flop / sec / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"full fp64 forward RELU_AUX_BIAS + backward DRELU_BGRAD at M=N=K={c.m} on the "
                      f"same inputs, {reps} rep(s), {sec:.2f} s each; host has {os.cpu_count()} logical CPUs"}


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
        elif args.only == "gelu":
            r = gelu_layer(W.LINEAR[2], st, wu, flush, dev)
        elif args.only == "mlp_step":
            r = mlp_training_step(W.SWIGLU[4], st, wu, flush, dev)
        elif args.only == "dswiglu":
            r = dswiglu_bwd(W.SWIGLU[5], st, wu, flush, dev)
        else:
            raise SystemExit(f"unknown --only {args.only}")
        print(json.dumps({"only": args.only, "result": r}))
        return

    c2 = W.LINEAR[2]
    t_start = time.time()
    r2 = linear_layer(c2, args.steps, args.warmup, flush, dev, with_clock=True)
    f2 = r2["fused"]
    fwd_tflops = f2["tflops_fwd"]
    line = {
        "metric": METRIC,
        "value": round(f2["tflops_step"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(f2["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "square ReLU linear layer, fp16 in / fp32 acc: fused RELU_AUX_BIAS forward "
                               "(X 4096x4096 . W 4096x4096 + bias) then fused DRELU_BGRAD backward "
                               "(dY . W^T masked by the forward relu_aux, + bgrad)",
                   "m": c2.m, "n": c2.n, "k": c2.k,
                   "cache": f"cold: steps rotate over {f2['input_sets']} copies of the inputs (more than the "
                            "256 MB Infinity Cache together)"},
        "timing": "4 blocks of steps/4 back-to-back steps per variant, one HIP event pair per block, "
                  "fused / unfused / torch blocks alternating; median/min/max are over the blocks",
        "ms_per_step_median": round(f2["step_ms_median"], 5),
        "ms_per_step_min": round(f2["step_ms_min"], 5), "ms_per_step_max": round(f2["step_ms_max"], 5),
        "pct_peak": round(100.0 * f2["tflops_step"] / PEAK_F16_TFLOPS, 2),
        "speedup_vs_unfused": round(r2["speedup_step"], 4),
        "unfused_ms_per_step": round(r2["unfused"]["step_ms"], 5),
        "torch_ms_per_step": round(r2["torch"]["step_ms"], 5),
        "speedup_vs_torch": round(r2["speedup_vs_torch"], 4),
        "fwd_ms": round(f2["fwd_ms"], 5), "bwd_ms": round(f2["bwd_ms"], 5),
        "roofline": {"bound": "mfma", "kernel": f2["fwd_info"].split("kernels=")[1],
                     "achieved": round(fwd_tflops, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fwd_tflops / PEAK_F16_TFLOPS, 4), "traffic": None,
                     "algorithmic_per_launch": f"{r2['flop_per_gemm']:.6g} FLOP (2*4096^3)",
                     "algorithmic_bytes_per_launch": ALGO_BYTES_SQ4096_FWD,
                     "avg_launch_ms": round(f2["fwd_ms"], 5),
                     "avg_launch_how": "20 back-to-back launches of the forward between one HIP event pair "
                                       "on the launch stream"},
    }
    line["clock_under_load"] = r2["clock"]
    tr = measured_traffic()
    if tr is not None:
        line["roofline"]["traffic"] = round(tr["traffic_bytes_per_launch"])
        line["roofline"]["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    if not args.no_large:
        large = {}
        s_l, w_l = max(3, args.steps // 4), max(1, args.warmup // 2)
        r3 = linear_layer(W.LINEAR[3], s_l, w_l, flush, dev)
        r3.pop("inputs")
        large["h200_fp16_65536x16384x8192"] = {
            "fused_fwd_tflops": round(r3["fused"]["tflops_fwd"], 1),
            "fused_bwd_tflops": round(r3["fused"]["tflops_bwd"], 1),
            "fwd_pct_peak": round(100 * r3["fused"]["tflops_fwd"] / PEAK_F16_TFLOPS, 2),
            "bwd_pct_peak": round(100 * r3["fused"]["tflops_bwd"] / PEAK_F16_TFLOPS, 2),
            "fused_fwd_ms": round(r3["fused"]["fwd_ms"], 4), "fused_bwd_ms": round(r3["fused"]["bwd_ms"], 4),
            "unfused_fwd_ms": round(r3["unfused"]["fwd_ms"], 4), "unfused_bwd_ms": round(r3["unfused"]["bwd_ms"], 4),
            "speedup_fwd": round(r3["speedup_fwd"], 4), "speedup_bwd": round(r3["speedup_bwd"], 4),
            "torch_step_ms": round(r3["torch"]["step_ms"], 4), "speedup_step_vs_torch": round(r3["speedup_vs_torch"], 4)}
        torch.cuda.empty_cache()
        r4 = swiglu_fwd(W.SWIGLU[4], args.steps, args.warmup, flush, dev)
        large["swiglu_fwd_bf16_M2048_H5120_I17408"] = {
            "fused_swiglu_tflops": round(r4["fused"]["tflops_swiglu"], 1),
            "swiglu_pct_peak": round(100 * r4["fused"]["tflops_swiglu"] / PEAK_F16_TFLOPS, 2),
            "down_gemm_tflops": round(r4["fused"]["tflops_down"], 1),
            "fused_swiglu_ms": round(r4["fused"]["swiglu_ms"], 4),
            "unfused_swiglu_ms": round(r4["unfused"]["swiglu_ms"], 4),
            "speedup_swiglu": round(r4["speedup_swiglu"], 4), "speedup_fwd_step": round(r4["speedup_step"], 4)}
        torch.cuda.empty_cache()
        r5 = dswiglu_bwd(W.SWIGLU[5], args.steps, args.warmup, flush, dev)
        large["dswiglu_bwd_bf16_M16384_H5120_I17408"] = {
            "fused_tflops": round(r5["fused"]["tflops"], 1),
            "pct_peak": round(100 * r5["fused"]["tflops"] / PEAK_F16_TFLOPS, 2),
            "fused_ms": round(r5["fused"]["ms"], 4), "unfused_ms": round(r5["unfused"]["ms"], 4),
            "speedup": round(r5["speedup"], 4)}
        torch.cuda.empty_cache()
        large["swiglu_fwd_bf16_M_sweep_H5120_I17408"] = swiglu_m_sweep(s_l, w_l, flush, dev)
        large["swiglu_mlp_training_step_bf16_M2048_H5120_I17408"] = mlp_training_step(W.SWIGLU[4], args.steps, args.warmup, flush, dev)
        torch.cuda.empty_cache()
        large["gelu_layer_fp16_4096x4096x4096"] = gelu_layer(W.LINEAR[2], args.steps, args.warmup, flush, dev)
        large["execute_overhead"] = execute_overhead(dev)
        large["autotune_vs_model"] = autotune_vs_model(s_l, w_l, flush, dev)
        line["configs"] = large
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(r2["inputs"], c2)
    line["wall_s"] = round(time.time() - t_start, 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
