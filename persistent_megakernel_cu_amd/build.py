"""Build libmk.so (the HIP library behind include/mk.h) in-tree for gfx950.

    python -m persistent_megakernel_cu_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Packed-FP32 instruction
selection is disabled for the device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmk.so")
SOURCES = ["mk_kernels.hip", "mk_api.cpp", "mk_plan.cpp"]
ARCH = os.environ.get("MK_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every source into libmk.so; returns the library path."""
    tmp = LIB + ".tmp"
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(os.path.dirname(PKG), "include"),
        "-x", "hip",
    ] + [os.path.join(CSRC, s) for s in SOURCES] + (extra_flags or []) + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmk.so")
    if verbose and r.stderr.strip():
        noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if noise:
            sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
