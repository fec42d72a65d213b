"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers in tests/host_sanitize/ are built with the sanitizers and run:
* the CPU oracle (oracle/oracle.cpp), every exported routine on small inputs with bad rows and
  parameters, degenerate sets, the fuzzy and uniform-draft variants;
* the C ABI's host code (the library sources compiled with host-side sanitizers; device code
  unchanged): the fan-out over its whole domain, workspace sizes, and every entry point's
  argument checks, which return before any launch (no GPU is touched).
A sanitizer report aborts the driver; the test requires a clean exit.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
# host-side only: each sanitizer flag of the HIP compile applies to the host pass
HIP_HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, env=None, timeout=600):
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    out = res.stdout + res.stderr
    assert res.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({res.returncode}):\n{out[-4000:]}"
    return out


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not present")
    return tmp_path_factory.mktemp("sanitize")


def test_oracle_under_sanitizers(workdir):
    exe = str(workdir / "oracle_driver")
    _run([CLANG, "-std=c++17", "-O1", "-g", *SAN, os.path.join(HERE, "oracle_driver.cpp"),
          os.path.join(ROOT, "oracle", "oracle.cpp"), "-o", exe, "-lpthread"])
    out = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert "calls clean" in out


def test_capi_host_code_under_sanitizers(workdir):
    hip = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not shutil.which(hip) and not os.path.exists(hip):
        pytest.skip("hipcc not present")
    csrc = os.path.join(ROOT, "lossless_speculative_sampling_amd", "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    objdir = workdir / "obj"
    objdir.mkdir()
    compile_cmd = [hip, "-c", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HIP_HOST_SAN,
                   "-I", os.path.join(ROOT, "include"), *srcs]
    res = subprocess.run(compile_cmd, capture_output=True, text=True, cwd=str(objdir), timeout=900)
    assert res.returncode == 0, res.stderr[-4000:]
    objs = sorted(str(objdir / f) for f in os.listdir(objdir) if f.endswith(".o"))
    exe = str(workdir / "capi_driver")
    _run([CLANG, "-std=c++17", "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
          "-D__HIP_PLATFORM_AMD__", os.path.join(HERE, "capi_driver.cpp"), *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    # the HIP runtime keeps allocations until exit: leak checking stays off for this driver
    out = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"}, timeout=120)
    assert ", 0 failures" in out
