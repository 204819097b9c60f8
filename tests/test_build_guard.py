"""CPU tests of the build's resource guard (no GPU work).

The 16x16x32 MFMA configurations issue their MFMAs as inline asm, whose hazards the compiler
does not track; they are correct only while the kernel has no scratch, spills or register
moves around them.  The build compiles every kernel with the compiler's resource-usage
remarks and refuses any kernel that uses scratch or spills.  These tests check the guard
itself on planted remarks, and the real figures of one compiled instantiation.
"""
import json
import os
import subprocess

import pytest

from dense_gemm_epilogues_amd import build as B


def remark(name, scratch=0, vspill=0, sspill=0):
    lines = [f"gemm_kernel.hpp:307:1: remark: Function Name: {name} [-Rpass-analysis=kernel-resource-usage]",
             "gemm_kernel.hpp:307:1: remark:     TotalSGPRs: 51 [-Rpass-analysis=kernel-resource-usage]",
             "gemm_kernel.hpp:307:1: remark:     VGPRs: 90 [-Rpass-analysis=kernel-resource-usage]",
             "gemm_kernel.hpp:307:1: remark:     AGPRs: 256 [-Rpass-analysis=kernel-resource-usage]",
             f"gemm_kernel.hpp:307:1: remark:     ScratchSize [bytes/lane]: {scratch} [-Rpass-analysis=kernel-resource-usage]",
             "gemm_kernel.hpp:307:1: remark:     Occupancy [waves/SIMD]: 1 [-Rpass-analysis=kernel-resource-usage]",
             f"gemm_kernel.hpp:307:1: remark:     SGPRs Spill: {sspill} [-Rpass-analysis=kernel-resource-usage]",
             f"gemm_kernel.hpp:307:1: remark:     VGPRs Spill: {vspill} [-Rpass-analysis=kernel-resource-usage]",
             "gemm_kernel.hpp:307:1: remark:     LDS Size [bytes/block]: 131072 [-Rpass-analysis=kernel-resource-usage]"]
    return "\n".join(lines) + "\n"


M16 = "_ZN2ep11gemm_kernelILi0ELi0ELi3ELi9ELi0EEEvNS_8GemmArgsE"
M32 = "_ZN2ep11gemm_kernelILi0ELi0ELi3ELi0ELi0EEEvNS_8GemmArgsE"


def test_asm_mfma_configurations_from_the_tile_table():
    assert B.asm_mfma_cfgs() == {9, 10, 11, 12}


def test_parser_reads_every_field():
    u = B.parse_resource_usage(remark(M16, scratch=12, vspill=3, sspill=1))
    assert u == {M16: {"sgprs": 51, "vgprs": 90, "agprs": 256, "scratch": 12, "sgpr_spill": 1, "vgpr_spill": 3,
                       "lds": 131072}}


@pytest.mark.parametrize("kw", [{"scratch": 16}, {"vspill": 2}, {"sspill": 4}])
def test_guard_refuses_spilling_asm_mfma_kernel(kw):
    usage = B.parse_resource_usage(remark(M32) + remark(M16, **kw))
    with pytest.raises(RuntimeError, match="inline-asm MFMA configuration"):
        B.check_resource_usage(usage)


def test_guard_refuses_any_spilling_kernel_and_missing_figures():
    with pytest.raises(RuntimeError, match="spilling kernel"):
        B.check_resource_usage(B.parse_resource_usage(remark(M32, vspill=1)))
    usage = B.parse_resource_usage(remark(M16))
    del usage[M16]["scratch"]
    with pytest.raises(RuntimeError, match="no scratch figure"):
        B.check_resource_usage(usage)
    assert B.check_resource_usage(B.parse_resource_usage(remark(M32) + remark(M16))) == 2


def test_one_compiled_instantiation_passes(tmp_path):
    """Compile the fp16 K x N RELU_AUX_BIAS unit (every tile configuration, whole-K and split-K
    fixup kernels) with the remarks: the 16x16 kernels are among them and none spills."""
    obj, usage = B._compile((os.path.join(B.CSRC, "gemm_inst.hip"), str(tmp_path / "g.o"),
                             ["-DEP_DT=0", "-DEP_LAY=0", "-DEP_EPI=3"]))
    names = list(usage)
    assert any("ELi9ELi0E" in n for n in names) and any("ELi10ELi0E" in n for n in names), names
    assert B.check_resource_usage(usage) == len(names) >= 22


def test_full_build_report_if_built():
    """The report the last build wrote covers every kernel of the library and passes."""
    if not os.path.exists(B.REPORT):
        pytest.skip("library not built here")
    usage = json.load(open(B.REPORT))
    assert len(usage) > 500
    assert B.check_resource_usage(usage) == len(usage)
