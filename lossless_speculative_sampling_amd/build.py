"""Builds libspecverify.so (the C-ABI HIP library) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libspecverify.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 instructions stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    # per-kernel register report, checked below
    "-Rpass-analysis=kernel-resource-usage",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def vgpr_spills(report: str) -> dict[str, int]:
    """Kernels whose VGPRs spill to scratch, from the compiler's resource-usage remarks.

    A spilled vector register is stored under the execution mask of the point where the
    compiler places the spill; when that point lies inside a branch taken by only some waves
    or lanes, the others lose the value.  The kernels here are written to fit their register
    budgets, so any spill is treated as a build error.
    """
    return _per_kernel(report, "VGPRs Spill:")


def scratch_users(report: str) -> dict[str, int]:
    """Kernels with private (scratch) memory per lane: an array indexed at run time, a call's
    stack frame or a spill.  Scratch has to be set up for every wave at launch, which the
    latency-bound calls here pay for, and none of their paths needs it; any is a build error."""
    return _per_kernel(report, "ScratchSize [bytes/lane]:")


# kernels whose resource report must be present (a missing report would let a spill through)
EXPECTED_KERNELS = ("fast_count_kernel", "fast_resolve_kernel", "fast_diverge_kernel", "generic_unit_kernel",
                    "finalize_kernel", "cache_lookup_kernel", "signpost_kernel")


def report_problems(report: str) -> list[str]:
    """What the compiler's resource report lacks: no per-kernel remarks at all, a kernel without
    its spill or scratch line, or an expected kernel without a report."""
    names, seen = [], {}
    name = None
    for line in report.splitlines():
        if "remark: Function Name:" in line:
            name = line.split("Function Name:")[1].split("[")[0].strip()
            names.append(name)
            seen[name] = set()
        elif "remark:" in line and name is not None:
            for key in ("VGPRs Spill:", "ScratchSize [bytes/lane]:"):
                if key in line:
                    seen[name].add(key)
    if not names:
        return ["no kernel-resource-usage remarks in the compiler output"]
    out = [f"{n}: no '{k}' line" for n in names for k in ("VGPRs Spill:", "ScratchSize [bytes/lane]:")
           if k not in seen[n]]
    for k in EXPECTED_KERNELS:
        if not any(k in n for n in names):
            out.append(f"no resource report for {k}")
    return out


def _per_kernel(report: str, key: str) -> dict[str, int]:
    found: dict[str, int] = {}
    name = None
    for line in report.splitlines():
        if "remark: Function Name:" in line:
            name = line.split("Function Name:")[1].split("[")[0].strip()
        elif "remark:" in line and key in line and name is not None:
            n = int(line.split(key)[1].split("[")[0])
            if n:
                found[name] = n
    return found


def build_library(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    out = res.stdout + res.stderr
    msg = "\n".join(l for l in out.splitlines() if noise not in l and "remark:" not in l and not l.startswith(" "))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msg}")
    problems = report_problems(out)
    if problems:
        raise RuntimeError("kernel resource report incomplete: " + "; ".join(problems[:8]))
    spills = vgpr_spills(out)
    if spills:
        raise RuntimeError(f"vector registers spill to scratch in: {spills}")
    scratch = scratch_users(out)
    if scratch:
        raise RuntimeError(f"kernels use scratch memory (bytes per lane): {scratch}")
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
    sys.exit(0)
