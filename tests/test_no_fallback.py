"""The product path has no fallback: without libep.so the binding raises instead of computing,
and nothing in the package reaches the oracle (which is test infrastructure only)."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "dense_gemm_epilogues_amd")


def run_without_library(code):
    env = dict(os.environ, EP_LIBRARY=os.path.join(ROOT, "no-such-dir", "libep.so"))
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                          stderr=subprocess.STDOUT, text=True, timeout=300)


def test_missing_library_raises_on_every_entry():
    code = """
import dense_gemm_epilogues_amd as ep
failures = 0
for call in (lambda: ep.lib(), lambda: ep.abi_version(), lambda: ep.describe_plan(256, 256, 256),
             lambda: ep.Plan(None, None, "DEFAULT")):
    try:
        call()
    except ImportError as e:
        assert "is not built" in str(e), e
        failures += 1
print("raised", failures)
"""
    r = run_without_library(code)
    assert r.returncode == 0 and "raised 4" in r.stdout, r.stdout[-2000:]


def test_package_never_imports_the_oracle():
    for name in sorted(os.listdir(PKG)):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(PKG, name)).read())
        for node in ast.walk(tree):
            mods = []
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), f"{name} imports the oracle"


def test_bench_uses_the_oracle_only_for_the_cpu_baseline():
    """bench.py imports the oracle inside its CPU-timing functions only."""
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    for fn in [n for n in tree.body if isinstance(n, ast.FunctionDef)]:
        uses = any(isinstance(n, ast.Import) and any(a.name == "oracle" for a in n.names) for n in ast.walk(fn))
        if uses:
            assert fn.name.startswith(("cpu_baseline", "cpu_oracle")), fn.name
    assert not any(isinstance(n, ast.Import) and any(a.name == "oracle" for a in n.names) for n in tree.body)


def test_oracle_is_independent_of_the_product():
    """The oracle imports numpy and scipy only: neither the library, its binding, torch nor the
    input generators (which both sides share)."""
    for name in sorted(os.listdir(os.path.join(ROOT, "oracle"))):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(ROOT, "oracle", name)).read())
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""] if node.level == 0 else []
            else:
                continue
            for m in mods:
                assert m.split(".")[0] in ("numpy", "scipy", "math", "fractions", "json", "os"), f"oracle/{name} imports {m}"
