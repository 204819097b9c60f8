"""Summaries of rocprofv3 output for this library's kernels.

  python -m dense_gemm_epilogues_amd.profiling stats DIR
      per-kernel call count and average duration from a `--kernel-trace --stats
      --output-format csv` run (reads *_kernel_stats.csv).
  python -m dense_gemm_epilogues_amd.profiling trace DIR
      per (kernel, grid size) call count and average duration from the kernel trace
      (reads *_kernel_trace.csv), so launches of one kernel at different shapes separate.
  python -m dense_gemm_epilogues_amd.profiling runs DIR KERNEL_SUBSTR [--grid G] [--min N]
      every run of at least N consecutive dispatches (in start-time order, no other kernel
      in between) of the kernel whose name contains KERNEL_SUBSTR, with its mean duration:
      picks out the back-to-back launches a benchmark times between one event pair.
  python -m dense_gemm_epilogues_amd.profiling counters PMC_DIR [PMC_DIR ...] --trace TRACE_DIR [--copy-bytes B]
      per (kernel, grid size) averages of every counter in the `--pmc` runs, with the
      sustained shader clock (GRBM_GUI_ACTIVE / XCDs / duration), the MFMA busy fraction
      (SQ_VALU_MFMA_BUSY_CYCLES / (cycles x SIMDs)) and the LDS bank-conflict fraction
      (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE), the L1 -> L2 read bytes and mean latency
      (TCP_TCC_READ_REQ_sum x 128, TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum), and
      with --copy-bytes B the HBM read and write rates from FETCH_SIZE / WRITE_SIZE runs that
      also recorded one device copy of B bytes (the counters' scale); durations come from
      the kernel trace.
  python -m dense_gemm_epilogues_amd.profiling traffic FETCH_DIR WRITE_DIR KERNEL_SUBSTR \
      --copy-bytes B [--grid G] [--out FILE]
      HBM bytes per launch of the kernel whose name contains KERNEL_SUBSTR (and, with
      --grid, whose grid size is G), from a `--pmc FETCH_SIZE` run and a `--pmc WRITE_SIZE`
      run (KiB per dispatch).  Each counter is scaled by what it reads for a plain device
      copy of B bytes recorded in the same run (the largest dispatch of the runtime's
      device-to-device copy kernel, __amd_rocclr_copyBuffer), and the result is tagged with the
      hash of the kernel sources it was measured on.

A traffic file is '#' comment lines (how it was made) followed by one JSON object;
read_record() parses it.  source_hash() is the hash of the HIP/C++ sources of libep.so; a stored traffic figure is
only valid while it matches.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

_HERE = os.path.dirname(os.path.abspath(__file__))


# the files whose text defines the fused GEMM kernels' device code (the planner, the C ABI
# and the elementwise kernels do not change what a counter run of a GEMM launch measures)
KERNEL_SOURCES = ("ep_internal.hpp", "gemm_inst.hip", "gemm_kernel.hpp", "normal_dist.hpp", "pair_sched.hpp")


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(_HERE, "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def read_record(path):
    with open(path) as f:
        return json.loads("".join(l for l in f if not l.startswith("#")))


def _find(d, pattern):
    hits = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return hits[0]


def kernel_stats(d):
    """[(name, calls, avg_ns, total_ns)] sorted by total time."""
    rows = list(csv.DictReader(open(_find(d, "*kernel_stats.csv"))))
    out = []
    for r in rows:
        out.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["TotalDurationNs"])))
    return sorted(out, key=lambda x: -x[3])


def kernel_trace(d):
    """[(name, grid, calls, avg_ns)] from the per-dispatch kernel trace."""
    rows = list(csv.DictReader(open(_find(d, "*kernel_trace.csv"))))
    acc = defaultdict(list)
    for r in rows:
        g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        acc[(r["Kernel_Name"], g)].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = [(k[0], k[1], len(v), sum(v) / len(v)) for k, v in acc.items()]
    return sorted(out, key=lambda x: -x[2] * x[3])


def dispatch_runs(d, kernel, grid=None, min_len=20):
    """[(first dispatch index, length, avg_ns)] for each run of >= min_len consecutive
    dispatches of one kernel (name contains `kernel`, grid size `grid` if given)."""
    rows = list(csv.DictReader(open(_find(d, "*kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    out, cur = [], []

    def close(i):
        if len(cur) >= min_len:
            out.append((i - len(cur), len(cur), sum(cur) / len(cur)))

    for i, r in enumerate(rows):
        g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        if kernel in r["Kernel_Name"] and (grid is None or g == grid):
            cur.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        else:
            close(i)
            cur = []
    close(len(rows))
    return out


def pmc_dispatches(d, counter):
    """[(kernel name, grid size, value)] per dispatch for one counter."""
    rows = list(csv.DictReader(open(_find(d, "*counter_collection.csv"))))
    return [(r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"]))
            for r in rows if r["Counter_Name"] == counter]


# MI355X: 8 XCDs of 32 CUs, 4 SIMDs per CU.  GRBM_GUI_ACTIVE counts busy cycles per XCD and
# rocprofv3 sums it over the XCDs; SQ_VALU_MFMA_BUSY_CYCLES sums over every SIMD.
XCDS, SIMDS = 8, 256 * 4


def counters(pmc_dirs, trace_dir, copy_bytes=0):
    """[(name, grid, n, {counter: mean}, derived)] for every kernel in the counter runs.

    With copy_bytes, FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled in each run by
    what they read for that run's largest device-to-device copy of copy_bytes bytes, and
    the HBM read / write rates are derived from them."""
    per = defaultdict(lambda: defaultdict(list))
    for d in pmc_dirs:
        disp = defaultdict(dict)
        for r in csv.DictReader(open(_find(d, "*counter_collection.csv"))):
            key = (r["Kernel_Name"], int(r["Grid_Size"]))
            disp[(key, r["Dispatch_Id"])][r["Counter_Name"]] = float(r["Counter_Value"])
        scale = {}
        if copy_bytes:
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                cal = [cs[c] for ((name, _), _), cs in disp.items() if CALIB_KERNEL in name and c in cs]
                if cal:
                    scale[c] = copy_bytes / (max(cal) * 1024.0)
        for (key, _), cs in disp.items():
            for c, v in cs.items():
                per[key][c].append(v)
                if c in scale:
                    per[key][c + "_bytes"].append(v * 1024.0 * scale[c])
    dur = {(n, g): avg for (n, g, _, avg) in kernel_trace(trace_dir)}
    out = []
    for key, cs in per.items():
        mean = {c: sum(v) / len(v) for c, v in cs.items()}
        der = {}
        t = dur.get(key)
        if t and "GRBM_GUI_ACTIVE" in mean:
            cyc = mean["GRBM_GUI_ACTIVE"] / XCDS
            der["duration_us"] = t / 1e3
            der["clock_GHz"] = cyc / t
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                der["mfma_busy"] = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMDS)
        if mean.get("SQ_LDS_IDX_ACTIVE"):
            der["lds_bank_conflict_frac"] = mean.get("SQ_LDS_BANK_CONFLICT", 0.0) / mean["SQ_LDS_IDX_ACTIVE"]
        if t:
            if "FETCH_SIZE_bytes" in mean:
                der["hbm_read_GBps"] = mean["FETCH_SIZE_bytes"] / t
            if "WRITE_SIZE_bytes" in mean:
                der["hbm_write_GBps"] = mean["WRITE_SIZE_bytes"] / t
        if mean.get("TCP_TCC_READ_REQ_sum"):
            # L1 -> L2 read requests (128-byte lines) and their mean latency in cycles
            der["l2_read_MB"] = mean["TCP_TCC_READ_REQ_sum"] * 128 / 1e6
            if "TCP_TCC_READ_REQ_LATENCY_sum" in mean:
                der["l2_read_latency_cycles"] = mean["TCP_TCC_READ_REQ_LATENCY_sum"] / mean["TCP_TCC_READ_REQ_sum"]
        out.append((key[0], key[1], max(len(v) for v in cs.values()), mean, der))
    return sorted(out, key=lambda x: -der_time(x))


def der_time(x):
    return x[4].get("duration_us", 0.0)


def _mean(rows, substr, grid=None):
    vals = [v for (k, g, v) in rows if substr in k and (grid is None or g == grid)]
    if not vals:
        raise KeyError(f"no dispatch of a kernel containing {substr!r}")
    return sum(vals) / len(vals), len(vals), next(k for (k, g, v) in rows if substr in k)


CALIB_KERNEL = "__amd_rocclr_copyBuffer"


def traffic(fetch_dir, write_dir, kernel, copy_bytes, grid=None):
    f = pmc_dispatches(fetch_dir, "FETCH_SIZE")
    w = pmc_dispatches(write_dir, "WRITE_SIZE")
    fk, fn, kname = _mean(f, kernel, grid)
    wk, wn, _ = _mean(w, kernel, grid)
    # the calibration copy is the runtime's device-to-device copy kernel (torch's dtype casts
    # also carry "copy" in their names and count differently)
    cf = max(v for (k, g, v) in f if CALIB_KERNEL in k)
    cw = max(v for (k, g, v) in w if CALIB_KERNEL in k)
    fetch_scale = copy_bytes / (cf * 1024.0)
    write_scale = copy_bytes / (cw * 1024.0)
    return {
        "kernel": kname,
        "grid": grid,
        "dispatches": [fn, wn],
        "fetch_kib_per_launch_raw": fk,
        "write_kib_per_launch_raw": wk,
        "copy_bytes": copy_bytes,
        "copy_fetch_kib_raw": cf,
        "copy_write_kib_raw": cw,
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "fetch_bytes_per_launch": fk * 1024.0 * fetch_scale,
        "write_bytes_per_launch": wk * 1024.0 * write_scale,
        "traffic_bytes_per_launch": fk * 1024.0 * fetch_scale + wk * 1024.0 * write_scale,
        "source_hash": source_hash(),
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    tr = sub.add_parser("trace")
    tr.add_argument("dir")
    ru = sub.add_parser("runs")
    ru.add_argument("dir")
    ru.add_argument("kernel")
    ru.add_argument("--grid", type=int, default=None)
    ru.add_argument("--min", type=int, default=20)
    c = sub.add_parser("counters")
    c.add_argument("pmc_dirs", nargs="+")
    c.add_argument("--trace", required=True)
    c.add_argument("--only", default="gemm_kernel")
    c.add_argument("--copy-bytes", type=int, default=0)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("kernel")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--grid", type=int, default=None)
    t.add_argument("--out")
    t.add_argument("--how", action="append", default=[],
                   help="command lines that produced the counter runs, kept as '#' lines")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        for name, calls, avg, tot in kernel_stats(a.dir):
            print(f"{calls:6d} calls  avg {avg / 1e3:11.2f} us  total {tot / 1e6:10.3f} ms  {name[:110]}")
    elif a.cmd == "counters":
        for name, grid, n, mean, der in counters(a.pmc_dirs, a.trace, a.copy_bytes):
            if a.only not in name:
                continue
            print(f"{name[:60]}  grid {grid}  dispatches {n}")
            print("    " + "  ".join(f"{k}={v:.4g}" for k, v in der.items()))
            print("    " + "  ".join(f"{k}={v:.4g}" for k, v in sorted(mean.items())))
    elif a.cmd == "runs":
        for first, n, avg in dispatch_runs(a.dir, a.kernel, a.grid, a.min):
            print(f"dispatch {first:7d}  run of {n:6d}  avg {avg / 1e3:11.2f} us")
    elif a.cmd == "trace":
        for name, grid, calls, avg in kernel_trace(a.dir):
            print(f"{calls:6d} calls  grid {grid:9d}  avg {avg / 1e3:11.2f} us  {name[:100]}")
    else:
        r = traffic(a.fetch_dir, a.write_dir, a.kernel, a.copy_bytes, a.grid)
        txt = json.dumps(r, indent=1)
        if a.out:
            with open(a.out, "w") as f:
                for line in a.how:
                    f.write("# " + line + "\n")
                f.write(txt + "\n")
        print(txt)
    return 0


if __name__ == "__main__":
    sys.exit(main())
