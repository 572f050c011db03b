"""The build's per-kernel resource check (adamw_optimizer_step_amd/build.py):
the compiler's resource-usage remarks are parsed, and a build fails when a
kernel uses scratch memory or when two waves of the persistent GEMM leave no
room on a SIMD for a wave of the AdamW update that may run beside it."""
import json
import os

import pytest

from adamw_optimizer_step_amd import build as B


def remarks(entries):
    # the shape of clang's -Rpass-analysis=kernel-resource-usage output
    out = []
    for name, vgprs, agprs, scratch in entries:
        out += [f"x.hip:1:1: remark: Function Name: {name} [-Rpass-analysis=kernel-resource-usage]",
                "    1 | __global__ void k() {", "      | ^",
                f"x.hip:1:1: remark:     TotalSGPRs: 80 [-Rpass-analysis=kernel-resource-usage]",
                f"x.hip:1:1: remark:     VGPRs: {vgprs} [-Rpass-analysis=kernel-resource-usage]",
                f"x.hip:1:1: remark:     AGPRs: {agprs} [-Rpass-analysis=kernel-resource-usage]",
                f"x.hip:1:1: remark:     ScratchSize [bytes/lane]: {scratch} [-Rpass-analysis=kernel-resource-usage]",
                f"x.hip:1:1: remark:     LDS Size [bytes/block]: 1024 [-Rpass-analysis=kernel-resource-usage]"]
    return "\n".join(out)


GEMM = "_ZN2ma11ns_gemm_dmaILi1ELb1ELi2ELi4ELb0ELb0EEEvNS_6NsArgsE"
ADAMW = "_ZN2ma12k_adamw_leanENS_8AdamArgsE"


def test_parse_resources_reads_every_kernel():
    r = B.parse_resources(remarks([(GEMM, 232, 0, 0), (ADAMW, 43, 0, 0)]))
    assert r == {GEMM: {"vgprs": 232, "agprs": 0, "scratch": 0, "lds": 1024},
                 ADAMW: {"vgprs": 43, "agprs": 0, "scratch": 0, "lds": 1024}}


@pytest.mark.parametrize("gemm_vgprs, ok", [(232, True), (225, True), (233, False), (236, False)])
def test_two_gemm_waves_leave_room_for_an_adamw_wave(gemm_vgprs, ok):
    # 43 VGPRs are allocated as 48: 2 x 232 + 48 = 512, the SIMD's file
    bad = B.check_resources(B.parse_resources(remarks([(GEMM, gemm_vgprs, 0, 0), (ADAMW, 43, 0, 0)])))
    assert (bad == []) == ok


def test_accumulation_registers_count_too():
    bad = B.check_resources(B.parse_resources(remarks([(GEMM, 200, 40, 0), (ADAMW, 43, 0, 0)])))
    assert bad and GEMM in bad[0]


def test_scratch_fails_the_build():
    bad = B.check_resources(B.parse_resources(remarks([(ADAMW, 43, 0, 16)])))
    assert bad and "scratch" in bad[0]


def test_the_built_library_met_the_budget():
    # written by the last build: every kernel of the library, within budget
    path = os.path.join(B.BUILD, "resources.json")
    if not os.path.exists(path):
        pytest.skip("no build in this tree")
    res = json.load(open(path))
    assert any(B.GEMM_KERNEL in k for k in res) and any(B.BESIDE_KERNEL in k for k in res)
    assert B.check_resources(res) == []
