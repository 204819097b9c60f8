"""Host-side logic of bench.py, on the CPU: the algorithmic byte count of the roofline kernel,
the committed traffic records (parsed, tagged with the current kernel sources, consistent with
the algorithmic bytes), the oracle-rate record, the whole-oracle timing helper on the
32 x 64 x 128 layer, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402
from dense_gemm_epilogues_amd import profiling  # noqa: E402


def test_algo_bytes_fwd_counts_each_operand_once():
    # X (m x k), W (k x n), bias (n) read once; Y (m x n) written once: fp16, 2 bytes each;
    # relu_aux: ceil(n / 32) uint32 words per row
    assert bench.algo_bytes_fwd(1, 1, 1) == 2 * 4 + 4
    assert bench.algo_bytes_fwd(65536, 8192, 16384) == 3556786176
    assert bench.algo_bytes_fwd(3, 33, 5) == 2 * (15 + 165 + 33 + 99) + 4 * 3 * 2


@pytest.mark.parametrize("name,m,n,k", [("traffic_gemm_relu_aux_bias_f16_KN_65536x8192x16384.txt", 65536, 8192, 16384),
                                        ("traffic_gemm_relu_aux_bias_f16_KN_4096.txt", 4096, 4096, 4096)])
def test_traffic_record_matches_the_current_sources(name, m, n, k):
    """The committed traffic records were taken on the kernel sources in the tree (else bench.py
    reports their traffic null), and their writes are the algorithmic ones."""
    rec = profiling.read_record(os.path.join(ROOT, "profiles", name))
    assert rec["source_hash"] == profiling.source_hash()
    assert bench.measured_traffic(os.path.join(ROOT, "profiles", name)) is not None
    algo = bench.algo_bytes_fwd(m, n, k)
    written = 2 * m * n + 4 * m * ((n + 31) // 32)
    assert abs(rec["write_bytes_per_launch"] - written) / written < 0.01
    # every operand byte is fetched at least once
    assert rec["fetch_bytes_per_launch"] >= algo - written
    assert rec["traffic_bytes_per_launch"] == pytest.approx(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])


def test_measured_traffic_is_none_for_a_missing_or_stale_record(tmp_path):
    assert bench.measured_traffic(str(tmp_path / "missing.txt")) is None
    stale = tmp_path / "stale.txt"
    stale.write_text("# made on other sources\n" + json.dumps({"source_hash": "0" * 16, "traffic_bytes_per_launch": 1}))
    assert bench.measured_traffic(str(stale)) is None


def test_oracle_rate_record():
    r = bench.oracle_rate(2e9, 8e12, 0.5, 3, "what", 0.25)
    assert r["value"] == pytest.approx(4e9 / 1e12)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["cores"] >= 1
    assert r["extrapolated_full_step_s"] == pytest.approx(2000.0)
    assert "extrapolated" in r["extrapolated_note"]


def test_cpu_oracle_full_linear_on_the_small_layer():
    c = W.LINEAR[1]
    r = bench.cpu_oracle_full_linear(W.linear_inputs(c, device="cpu"), c, min_s=0.0)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["seconds_per_step"] > 0
    assert r["value"] == pytest.approx(4.0 * c.m * c.n * c.k / r["seconds_per_step"] / 1e12)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
