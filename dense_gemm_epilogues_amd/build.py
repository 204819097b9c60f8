"""Build libep.so (the C-ABI library with every HIP kernel) for gfx950 with hipcc.

Usage: python -m dense_gemm_epilogues_amd.build   (or __graft_entry__.build()).
Objects go to dense_gemm_epilogues_amd/_build/, the library to
dense_gemm_epilogues_amd/libep.so.  The fused-GEMM template is compiled once per
(dtype, B layout, epilog) in parallel.

Resource guard: every object is compiled with the compiler's kernel-resource-usage remarks,
and the build fails if any kernel uses scratch memory or spills registers.  For the
configurations that issue their MFMAs as inline asm (16x16x32, whose hazards the compiler
does not track), a spill or register move around the MFMAs can make them read accumulators
before their results land, so such a build must never reach a GPU; for the others a spill
is a performance bug.  The per-kernel figures go to _build/resource_usage.json.
"""
import json
import os
import re
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
REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
REPORT = os.path.join(BUILD, "resource_usage.json")

_FIELDS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
           "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds"}


def parse_resource_usage(text):
    """{mangled kernel name: {field: int}} from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*?): (-?\d+)\s", line + " ")
        if m and cur is not None and m.group(1) in _FIELDS:
            cur[_FIELDS[m.group(1)]] = int(m.group(2))
    return out


def asm_mfma_cfgs():
    """Tile configurations whose MFMAs are inline asm: the kTileCfgs rows of ep_internal.hpp with
    a 16-wide MFMA block (the field after vst)."""
    text = open(os.path.join(CSRC, "ep_internal.hpp")).read()
    table = text[text.index("kTileCfgs[kNumTileCfgs] = {"):]
    table = table[:table.index("};")]
    rows = [[int(v) for v in re.findall(r"\d+", r)] for r in re.findall(r"\{((?:\s*\d+,)+)\s*\"", table)]
    return {i for i, r in enumerate(rows) if r[6] == 16}


def check_resource_usage(usage, asm_cfgs=None):
    """Raise RuntimeError naming every kernel that uses scratch or spills registers (see the
    module docstring); returns the number of kernels checked."""
    asm_cfgs = asm_mfma_cfgs() if asm_cfgs is None else asm_cfgs
    bad = []
    for name, u in usage.items():
        missing = [f for f in ("scratch", "vgpr_spill", "sgpr_spill") if f not in u]
        if missing:
            bad.append(f"{name}: no {', '.join(missing)} figure in the compiler's remarks")
            continue
        if u["scratch"] or u["vgpr_spill"] or u["sgpr_spill"]:
            m = re.search(r"gemm_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E", name)
            why = ("inline-asm MFMA configuration: spills or moves around the MFMAs break their hazard "
                   "handling" if m and int(m.group(4)) in asm_cfgs else "spilling kernel")
            bad.append(f"{name}: scratch {u['scratch']} B/lane, VGPR spill {u['vgpr_spill']}, "
                       f"SGPR spill {u['sgpr_spill']} ({why})")
    if bad:
        raise RuntimeError("resource guard failed:\n  " + "\n  ".join(bad))
    return len(usage)


def _compile(args):
    src, obj, defines = args
    cmd = [HIPCC] + FLAGS + defines + REMARKS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    return obj, parse_resource_usage(r.stdout)


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
    tasks.append((os.path.join(CSRC, "static_scratch.hip"), os.path.join(BUILD, "static_scratch.o"), []))
    tasks.append((os.path.join(CSRC, "ep_api.cpp"), os.path.join(BUILD, "ep_api.o"), []))
    jobs = jobs or min(16, os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        done = list(ex.map(_compile, tasks))
    objs = [o for o, _ in done]
    usage = {}
    for _, u in done:
        usage.update(u)
    with open(REPORT, "w") as f:
        json.dump(usage, f, indent=0, sort_keys=True)
    n = check_resource_usage(usage)
    if verbose:
        print(f"resource guard: {n} kernels, none uses scratch or spills")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


HOSTSAN_LIB = os.path.join(BUILD, "libep_hostsan.so")


def build_host_sanitized(verbose=False):
    """Host-sanitizer build of the C ABI for the CPU tests: ep_api.cpp (validation, planning,
    dispatch; host code only) compiled by g++ with AddressSanitizer and UndefinedBehavior-
    Sanitizer, linked with the kernel objects of the last build() (not instrumented).  Load it
    with EP_LIBRARY pointing here and the sanitizer runtimes in LD_PRELOAD."""
    src = os.path.join(CSRC, "ep_api.cpp")
    obj = os.path.join(BUILD, "ep_api_hostsan.o")
    objs = sorted(os.path.join(BUILD, f) for f in os.listdir(BUILD) if f.startswith("gemm_") and f.endswith(".o"))
    objs += [os.path.join(BUILD, "elementwise.o"), os.path.join(BUILD, "static_scratch.o")]
    if not all(os.path.exists(o) for o in objs) or len(objs) < 3:
        raise RuntimeError("run build() first: the sanitized library links its kernel objects")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    gxx_compile = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"), "-I", CSRC, "-I", INCLUDE, "-c", src, "-o", obj] + san
    r = subprocess.run(gxx_compile, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host-sanitizer compile failed:\n{r.stdout}")
    gxx_link = ["g++", "-shared", "-o", HOSTSAN_LIB, obj] + objs + ["-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")] + san
    r = subprocess.run(gxx_link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host-sanitizer link failed:\n{r.stdout}")
    if verbose:
        print(f"built {HOSTSAN_LIB}")
    return HOSTSAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
