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
