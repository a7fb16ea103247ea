"""Builds libsdv.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "sdv.hip"), os.path.join(PKG, "csrc", "commit.hip"),
           os.path.join(PKG, "csrc", "sdcp_uniforms.cpp")]
DEPENDS = SOURCES + [os.path.join(PKG, "csrc", "sdv_device.hpp"), os.path.join(PKG, "csrc", "split.hpp"),
                     os.path.join(ROOT, "include", "sdv.h")]
LIBRARY = os.path.join(PKG, "libsdv.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # packed fp32 instructions stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build_library(out: str = LIBRARY, verbose: bool = False) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, f"-I{os.path.join(ROOT, 'include')}", *SOURCES, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    if verbose and res.stderr:
        print(res.stderr)
    os.replace(tmp, out)
    return out


def is_stale(path: str = LIBRARY) -> bool:
    if not os.path.exists(path):
        return True
    t = os.path.getmtime(path)
    return any(os.path.getmtime(d) > t for d in DEPENDS)


if __name__ == "__main__":
    print(build_library(verbose=True))
