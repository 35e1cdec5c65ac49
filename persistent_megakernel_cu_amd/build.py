"""Build libmk.so (the HIP library behind include/mk.h) in-tree for gfx950.

    python -m persistent_megakernel_cu_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Every translation unit is
compiled to an object in _build/ (in parallel; the kernel instances are the
builds of csrc/mk_inst.hip with their template parameters as defines), then
linked into libmk.so.  Packed-FP32 instruction selection is disabled for the
device code.

The same call builds libmkcheck.so (host code only, g++): the planner plus the
address walk of csrc/mk_check.cpp, which the CPU tests use to replay a plan's
tape through the kernels' own index helpers.
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
LIB = os.path.join(PKG, "libmk.so")
CHECK_LIB = os.path.join(PKG, "libmkcheck.so")
OBJ_DIR = os.path.join(ROOT, "_build")
ARCH = os.environ.get("MK_OFFLOAD_ARCH", "gfx950")

# Kernel instances (query heads per kv head G, head_dim, batched, query heads
# per attention task GT (0: both variants, chosen at run time), flags: 1 trace
# stamps, 2 partial-input down projection).  Each instance carries only the
# code its plans run; the library picks one per plan (mk_kernels.hip).
INSTANCES = ([(g, 64, 0, gt, f) for f in (0, 2) for g in (1, 2, 4) for gt in sorted({1, g})]
             + [(g, 64, 0, 0, 1) for g in (1, 2, 4)]
             + [(g, 128, 0, 0, 0) for g in (1, 2, 4)]
             + [(g, 64, 1, 0, f) for f in (0, 1) for g in (1, 2, 4)])
UNITS = ([("mk_kernels", "mk_kernels.hip", []), ("mk_api", "mk_api.cpp", []), ("mk_plan", "mk_plan.cpp", []),
          ("conv_kernels", "conv_kernels.hip", []), ("w2a8", "w2a8.hip", [])]
         + [(f"mk_inst_{g}_{d}_{b}_{gt}_{f}", "mk_inst.hip",
             [f"-DMK_INST_G={g}", f"-DMK_INST_D={d}", f"-DMK_INST_B={b}", f"-DMK_INST_GT={gt}", f"-DMK_INST_F={f}"])
            for (g, d, b, gt, f) in INSTANCES])


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every source into libmk.so; returns the library path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    cc = hipcc()
    extra = extra_flags or []

    def compile_unit(u):
        name, src, defs = u
        obj = os.path.join(OBJ_DIR, name + ".o")
        cmd = [cc] + common_flags() + defs + extra + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        return name, obj, cmd, r

    def build_check():
        tmp = CHECK_LIB + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
               "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, "mk_check.cpp"),
               os.path.join(CSRC, "mk_plan.cpp"), "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode == 0:
            os.replace(tmp, CHECK_LIB)
        return cmd, r

    with ThreadPoolExecutor(max_workers=jobs()) as ex:
        check = ex.submit(build_check)
        results = list(ex.map(compile_unit, UNITS))
        ccmd, cres = check.result()
    if verbose:
        print(" ".join(ccmd), flush=True)
    if cres.returncode != 0:
        sys.stderr.write(cres.stdout + cres.stderr)
        raise RuntimeError("g++ failed building libmkcheck.so")
    failed = False
    for name, obj, cmd, r in results:
        if verbose:
            print(" ".join(cmd), flush=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            failed = True
    if failed:
        raise RuntimeError("hipcc failed building libmk.so")
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [obj for _, obj, _, _ in results]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed linking libmk.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
