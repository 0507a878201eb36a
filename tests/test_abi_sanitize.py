"""The C-ABI layer's host code under AddressSanitizer and
UndefinedBehaviorSanitizer: api.cpp is compiled with both (host side only),
linked with the library's kernel objects into tests/sanitize/abi_driver.cpp,
and every entry point is driven through its validation and workspace
arithmetic, including sizes at the int32 limits.  CPU only: without a GPU a
call that passes validation ends at the kernel launch."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp4_routed_expert_mxfp4_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
KERNEL_OBJS = ["combine_norm", "decode", "decode_cb3", "decode_mt", "prefill", "route_permute", "router_gate"]
# host-side sanitizers only: each flag is scoped to the host compilation
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_abi_host_code_under_sanitizers(tmp_path):
    objs = [os.path.join(BUILD, f"moe_{n}.hip.o") for n in KERNEL_OBJS]
    if not os.path.exists(_hipcc()) or not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's kernel objects are not built (python fp4_routed_expert_mxfp4_amd/build.py)")
    hipcc = _hipcc()
    api_o, drv_o, exe = str(tmp_path / "api.o"), str(tmp_path / "driver.o"), str(tmp_path / "abi_driver")
    common = ["-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC] + SANITIZE
    _run([hipcc, "-x", "hip", "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o, "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + common)
    _run([hipcc, "-c", os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", drv_o] + common)
    _run([hipcc, "-o", exe, drv_o, api_o] + objs + ["--offload-arch=gfx950"] + SANITIZE)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    report = r.stdout + r.stderr
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
    assert r.returncode == 0 and "OK: 0 mismatches" in r.stdout, report
