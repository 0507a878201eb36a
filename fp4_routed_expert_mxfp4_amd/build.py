"""Builds the gfx950 shared libraries in-tree with hipcc.

  fp4_routed_expert_mxfp4_amd/libmoe_fp4.so  the C-ABI MoE library (include/moe_fp4.h)
  gen/libmoe_gen.so                          the device filler of the synthetic inputs and the
                                             benchmark's streaming-read probe

Every HIP translation unit is compiled with packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

LIB_MOE = os.path.join(PKG, "libmoe_fp4.so")
LIB_GEN = os.path.join(ROOT, "gen", "libmoe_gen.so")
BUILD_INFO = os.path.join(PKG, "build_info.json")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build")
    return p


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), "-x", "hip", "-c", src, "-o", obj] + COMMON
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp] + objs + [f"--offload-arch={ARCH}", "-fPIC"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {out} failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 8) -> list[str]:
    os.makedirs(BUILD, exist_ok=True)
    moe_srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    gen_srcs = [os.path.join(ROOT, "gen", f) for f in ("fill.hip", "probe.hip")]
    units = [(s, os.path.join(BUILD, "moe_" + os.path.basename(s) + ".o")) for s in moe_srcs]
    units += [(s, os.path.join(BUILD, "gen_" + os.path.basename(s) + ".o")) for s in gen_srcs]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda u: _compile(*u), units))
    _link([o for s, o in units if os.path.basename(o).startswith("moe_")], LIB_MOE)
    _link([o for s, o in units if os.path.basename(o).startswith("gen_")], LIB_GEN)
    _write_build_info(moe_srcs + gen_srcs)
    return [LIB_MOE, LIB_GEN]


def _write_build_info(srcs: list[str]) -> None:
    """Records what the libraries were built from (the git commit when a
    checkout is present, and a hash of every source) beside them."""
    import hashlib
    import json
    h = hashlib.sha256()
    for s in sorted(srcs) + sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))):
        h.update(os.path.relpath(s, ROOT).encode())
        with open(s, "rb") as f:
            h.update(f.read())
    info = {"sources_sha256": h.hexdigest(), "arch": ARCH}
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=20)
        d = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"], capture_output=True,
                           text=True, timeout=20)
        if r.returncode == 0:
            info["git_head"] = r.stdout.strip()
            info["uncommitted_changes"] = bool(d.stdout.strip())
    except (OSError, subprocess.SubprocessError):
        pass
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f, indent=1)


if __name__ == "__main__":
    for p in build():
        print(p)
