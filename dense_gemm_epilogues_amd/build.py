"""Build libep.so (the C-ABI library with every HIP kernel) for gfx950 with hipcc.

Usage: python -m dense_gemm_epilogues_amd.build   (or __graft_entry__.build()).
Objects go to dense_gemm_epilogues_amd/_build/, the library to
dense_gemm_epilogues_amd/libep.so.  The fused-GEMM template is compiled once per
(dtype, B layout, epilog) in parallel.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libep.so")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops in device code
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", CSRC, "-I", INCLUDE,
]
N_EPI = 11


def _compile(args):
    src, obj, defines = args
    cmd = [HIPCC] + FLAGS + defines + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    return obj


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    tasks = []
    inst = os.path.join(CSRC, "gemm_inst.hip")
    # layouts 0/1: A M x K with B K x N / N x K, every epilog; 2/3: A given K x M, DEFAULT only
    for dt in (0, 1):
        for lay in (0, 1, 2, 3):
            for epi in (range(N_EPI) if lay < 2 else (0,)):
                obj = os.path.join(BUILD, f"gemm_{dt}_{lay}_{epi}.o")
                tasks.append((inst, obj, [f"-DEP_DT={dt}", f"-DEP_LAY={lay}", f"-DEP_EPI={epi}"]))
    tasks.append((os.path.join(CSRC, "elementwise.hip"), os.path.join(BUILD, "elementwise.o"), []))
    tasks.append((os.path.join(CSRC, "ep_api.cpp"), os.path.join(BUILD, "ep_api.o"), []))
    jobs = jobs or min(16, os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, tasks))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
