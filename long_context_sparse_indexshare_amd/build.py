"""Builds libisa.so (the HIP kernels and the C ABI) for gfx950, in place.

    python -m long_context_sparse_indexshare_amd.build

Each source compiles to its own object (in parallel), so a source can carry
code-generation flags of its own; the objects are then linked into one
shared library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libisa.so")
# attainable-peak probes that the benchmark reports beside the published peaks
# (measurement support; not linked into libisa.so)
PEAKS_SRC = os.path.join(PKG, "peaks", "peaks.hip")
PEAKS_LIB = os.path.join(PKG, "peaks", "libisa_peaks.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 math stays off: only scalar fp32 VALU forms are emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

# MFMA results in VGPRs where they fit: the indexer's int32 results feed VALU
# math at once, and the per-query attention kernel's loop-carried accumulators
# otherwise travel between AGPRs and VGPRs on every tile (several hundred
# accumulator moves per tile); kernels that need more than 256 registers still
# place the rest in AGPRs.
PER_FILE = {
    "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}

NOISE = "is not a recognized feature for this target"


def sources() -> list:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def compile_command(src: str, obj: str) -> list:
    return ["hipcc", *COMMON, *PER_FILE.get(os.path.basename(src), []),
            "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]


def link_command(objs: list, out: str) -> list:
    return ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd: list, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (res.stderr or "").splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for f in [ex.submit(_run, compile_command(s, o), verbose) for s, o in zip(srcs, objs)]:
            f.result()
    tmp = LIB + ".tmp"
    _run(link_command(objs, tmp), verbose)
    os.replace(tmp, LIB)
    ptmp = PEAKS_LIB + ".tmp"
    _run(["hipcc", *COMMON, "-shared", PEAKS_SRC, "-o", ptmp], verbose)
    os.replace(ptmp, PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
