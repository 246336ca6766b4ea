"""Compile the C-ABI library libw4a16.so for gfx950 (in-tree).

    python -m int4_weight_only_03_amd.build

Each source is compiled to an object under _build/ and the objects are linked
into int4_weight_only_03_amd/libw4a16.so.  The host quantizer is compiled
without FMA contraction so that it rounds exactly as its stated fp32 steps.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libw4a16.so")
ARCH = "gfx950"

DEVICE_SOURCES = ["gemv.hip", "gemv_mfma.hip", "tile.hip", "split.hip", "grouped.hip",
                  "small_packed.hip", "read_floor.hip", "skinny.hip", "tile_mx.hip"]
HOST_SOURCES = ["w4a16_api.cpp", "w4a16_io.cpp"]
# per-source options: the split path's MFMA results stay in VGPRs (the scale
# FMAs read them directly, no accumulator-register copies); so do the tiled
# kernel's block sums, which are added to running totals in VGPRs
EXTRA = {"split.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "tile.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: cannot build the gfx950 library")


COMMON = [
    "-std=c++17",
    "-O3",
    "-fPIC",
    f"--offload-arch={ARCH}",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return r


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source (in parallel) and link libw4a16.so; returns the library path."""
    from concurrent.futures import ThreadPoolExecutor

    cc = hipcc()
    os.makedirs(OBJ, exist_ok=True)
    cmds, objs = [], []
    for src in HOST_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        cmds.append([cc, *COMMON, "-ffp-contract=off", "-fno-fast-math", "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in DEVICE_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        cmds.append([cc, *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src),
                     "-o", obj])
        objs.append(obj)
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()  # re-raises the first failed compile
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
