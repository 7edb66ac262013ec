"""Build the HIP library libmoe_w4a16.so in-tree with hipcc for gfx950."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_w4a16.so")
SOURCES = ["api.cpp", "route_pack.hip", "prepare.hip", "decode.hip", "gemm.hip", "router.hip", "requant.hip", "static_workspace.hip"]
HEADERS = ["layout.hpp", "device.hpp", "kernels.hpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the library)")


def flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-munsafe-fp-atomics",
        # packed fp32 VALU ops are kept out of the device code on this platform
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def build(verbose: bool = False) -> str:
    """Compile every source into LIB (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags() + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    lines = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
