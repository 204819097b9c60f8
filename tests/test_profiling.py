"""CPU tests of the rocprofv3 summaries (dense_gemm_epilogues_amd.profiling) on small
hand-made CSV files in rocprofv3's column layout: per-kernel averages, the derived clock,
MFMA busy fraction, LDS bank-conflict fraction and the HBM rates scaled by the calibration
copy recorded in the same counter run."""
import csv
import os

import pytest

from dense_gemm_epilogues_amd import profiling as P

GEMM = "void ep::gemm_kernel<0, 0, 3, 11, 0>(ep::GemmArgs)"
COPY = "__amd_rocclr_copyBuffer"


def write_trace(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "t_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp", "End_Timestamp"])
        for name, grid, start, end in rows:
            w.writerow([name, grid, 1, 1, start, end])


def write_pmc(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for disp, name, grid, counter, value in rows:
            w.writerow([disp, name, grid, counter, value])


def test_counters_derived_values(tmp_path):
    # two dispatches of 100 us each; 8 XCDs at 1.5 GHz -> GRBM_GUI_ACTIVE = 8 * 150000
    write_trace(str(tmp_path / "tr"), [(GEMM, 262144, 0, 100_000), (GEMM, 262144, 200_000, 300_000)])
    cyc = 150_000
    write_pmc(str(tmp_path / "a"), [
        (1, GEMM, 262144, "GRBM_GUI_ACTIVE", 8 * cyc), (1, GEMM, 262144, "SQ_VALU_MFMA_BUSY_CYCLES", 0.75 * cyc * 1024),
        (2, GEMM, 262144, "GRBM_GUI_ACTIVE", 8 * cyc), (2, GEMM, 262144, "SQ_VALU_MFMA_BUSY_CYCLES", 0.75 * cyc * 1024),
        (3, GEMM, 262144, "SQ_LDS_BANK_CONFLICT", 10.0), (3, GEMM, 262144, "SQ_LDS_IDX_ACTIVE", 400.0)])
    # FETCH_SIZE: the copy of 1 MiB reads 512 KiB on the counter (scale 2); the GEMM reads 1000 KiB
    write_pmc(str(tmp_path / "f"), [(1, COPY, 4096, "FETCH_SIZE", 512.0), (2, GEMM, 262144, "FETCH_SIZE", 1000.0)])
    write_pmc(str(tmp_path / "w"), [(1, COPY, 4096, "WRITE_SIZE", 1024.0), (2, GEMM, 262144, "WRITE_SIZE", 300.0)])
    out = P.counters([str(tmp_path / d) for d in ("a", "f", "w")], str(tmp_path / "tr"), copy_bytes=1 << 20)
    gemm = [o for o in out if o[0] == GEMM][0]
    der = gemm[4]
    assert der["duration_us"] == pytest.approx(100.0)
    assert der["clock_GHz"] == pytest.approx(1.5)
    assert der["mfma_busy"] == pytest.approx(0.75)
    assert der["lds_bank_conflict_frac"] == pytest.approx(0.025)
    # 1000 KiB * 2 = 2048000 bytes in 100 us -> 20.48 GB/s; writes scale 1: 307200 bytes -> 3.072 GB/s
    assert der["hbm_read_GBps"] == pytest.approx(2048000 / 100_000)
    assert der["hbm_write_GBps"] == pytest.approx(307200 / 100_000)


def test_counters_without_calibration_has_no_rates(tmp_path):
    write_trace(str(tmp_path / "tr"), [(GEMM, 64, 0, 1000)])
    write_pmc(str(tmp_path / "f"), [(1, GEMM, 64, "FETCH_SIZE", 10.0)])
    der = P.counters([str(tmp_path / "f")], str(tmp_path / "tr"), copy_bytes=1 << 20)[0][4]
    assert "hbm_read_GBps" not in der and "hbm_write_GBps" not in der


def test_dispatch_runs_split_by_other_kernels(tmp_path):
    rows = [(GEMM, 8, 10 * i, 10 * i + 5) for i in range(25)] + [("other", 1, 300, 301)] + \
           [(GEMM, 8, 400 + 10 * i, 400 + 10 * i + 7) for i in range(20)]
    write_trace(str(tmp_path / "tr"), rows)
    runs = P.dispatch_runs(str(tmp_path / "tr"), "gemm_kernel", 8, 20)
    assert [(n, avg) for (_, n, avg) in runs] == [(25, 5.0), (20, 7.0)]
