"""The C ABI's host tests under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The validation path of ep_plan / ep_execute / ep_free / ep_plan_info and the planner behind
ep_plan_describe are host code: they are built a second time with both sanitizers
(build.build_host_sanitized, g++), loaded through the binding's EP_LIBRARY override, and
tests/test_abi_host.py and tests/test_planner_host.py run against it in a child process with
the sanitizer runtimes preloaded.  Any sanitizer report aborts the child.  (Reading an
out-of-range value from an enum-typed field was one such report, now fixed by reading the
raw int.)
"""
import os
import subprocess
import sys

import pytest

from dense_gemm_epilogues_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], stdout=subprocess.PIPE, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_abi_host_tests_under_asan_and_ubsan():
    if not os.path.exists(os.path.join(B.BUILD, "elementwise.o")):
        pytest.skip("library objects not built here")
    asan, ubsan = runtime("libasan.so"), runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = B.build_host_sanitized()
    env = dict(os.environ, EP_LIBRARY=lib, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = subprocess.run([sys.executable, "-c", "import dense_gemm_epilogues_amd as ep; ep.lib(); print(ep.library_path)"],
                           cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert probe.returncode == 0 and probe.stdout.strip().endswith(os.path.basename(lib)), probe.stdout[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_host.py"), os.path.join(ROOT, "tests", "test_planner_host.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    out = r.stdout
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and " passed" in out, out[-4000:]
