"""The build's resource checks: spills and scratch memory are build errors (CPU only)."""
from lossless_speculative_sampling_amd import build

REPORT = """\
k.hip:1:1: remark: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]
k.hip:1:1: remark:     VGPRs: 64 [-Rpass-analysis=kernel-resource-usage]
k.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:9:1: remark: Function Name: _Z3barPf [-Rpass-analysis=kernel-resource-usage]
k.hip:9:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]
k.hip:9:1: remark:     ScratchSize [bytes/lane]: 168 [-Rpass-analysis=kernel-resource-usage]
k.hip:9:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]
"""


def test_spills_and_scratch_are_reported_per_kernel():
    assert build.vgpr_spills(REPORT) == {"_Z3barPf": 3}
    assert build.scratch_users(REPORT) == {"_Z3barPf": 168}


def test_clean_report_has_no_findings():
    clean = "\n".join(l for l in REPORT.splitlines() if "_Z3bar" not in l and "k.hip:9" not in l)
    assert build.vgpr_spills(clean) == {} and build.scratch_users(clean) == {}


def test_missing_report_is_a_problem():
    assert build.report_problems("") == ["no kernel-resource-usage remarks in the compiler output"]
    # a kernel whose spill line is missing, and the expected kernels absent
    partial = "\n".join(l for l in REPORT.splitlines() if "VGPRs Spill" not in l or "k.hip:1" not in l)
    probs = build.report_problems(partial)
    assert "_Z3fooPf: no 'VGPRs Spill:' line" in probs
    assert any("fast_count_kernel" in p for p in probs)


def test_full_report_of_the_expected_kernels_is_clean():
    lines = []
    for i, k in enumerate(build.EXPECTED_KERNELS):
        lines += [f"k.hip:{i}:1: remark: Function Name: _ZN2sv4fast{k}E [-Rpass-analysis=kernel-resource-usage]",
                  f"k.hip:{i}:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
                  f"k.hip:{i}:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]"]
    assert build.report_problems("\n".join(lines)) == []
