"""Compile the HIP library (libkd.so) for gfx950 with hipcc, in-tree.

    python -m bandwidth_bound_transformer_amd.build

Every call recompiles.  The library is written next to this file, so the
Python binding loads it from the package directory.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkd.so")
SOURCES = [os.path.join(PKG, "csrc", "kd_api.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libkd.so")
    return path


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-shared",
        "-fPIC",
        # keep packed-FP32 instructions out of the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"),
        "-I", os.path.join(PKG, "csrc"),
        "-o", tmp,
        *SOURCES,
    ]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        sys.stderr.write(res.stdout)
        sys.stderr.write("\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l) + "\n")
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
