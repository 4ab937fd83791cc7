"""Build ``libmoe.so`` (the HIP kernels and the C-ABI of include/moe.h) for gfx950.

Usage: ``python -m expert_token_routing_amd.build_lib`` (or ``build()``).
Compiles every ``csrc/*.hip`` with hipcc in parallel and links one shared
library next to this file; ``calib/*.hip`` (counter calibration,
include/moe_calib.h) becomes ``libmoe_calib.so`` beside it. Always recompiles.
"""
from __future__ import annotations

import os
import pathlib
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libmoe.so"
CALIB_LIB = PKG / "libmoe_calib.so"
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-command-line-argument",
    # keep the compiler from forming packed float32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{ROOT / 'include'}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(map(str, cmd)) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False, jobs: int | None = None) -> pathlib.Path:
    cc = hipcc()
    BUILD.mkdir(exist_ok=True)
    sources = sorted(CSRC.glob("*.hip"))
    calib = sorted((PKG / "calib").glob("*.hip"))
    objs = [BUILD / (s.stem + ".o") for s in sources]
    calib_objs = [BUILD / ("calib_" + s.stem + ".o") for s in calib]

    def compile_one(pair):
        src, obj = pair
        out = _run([cc, *COMMON_FLAGS, "-c", str(src), "-o", str(obj)])
        if verbose and out.strip():
            print(out)
        return obj

    jobs = jobs or min(len(sources) + len(calib), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(compile_one, zip(sources + calib, objs + calib_objs)))
    for lib, lib_objs in ((LIB, objs), (CALIB_LIB, calib_objs)):
        tmp = lib.with_suffix(".so.tmp")
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, lib_objs)])
        os.replace(tmp, lib)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
