"""Build ``libmoe.so`` (the HIP kernels and the C-ABI of include/moe.h) for gfx950.

Usage: ``python -m expert_token_routing_amd.build_lib`` (or ``build()``).
Compiles every ``csrc/*.hip`` with hipcc in parallel and links one shared
library next to this file; ``calib/*.hip`` (counter calibration,
include/moe_calib.h) becomes ``libmoe_calib.so`` beside it. Always recompiles.
"""
from __future__ import annotations

import os
import pathlib
import re
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


_SGPR = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")


def _sgprs(text: str) -> set:
    out = set()
    for a, b, one in _SGPR.findall(text):
        out.update(range(int(a), int(b) + 1) if a else [int(one)])
    return out


def vmem_sgpr_hazards(asm: str, window: int = 5) -> list:
    """Direct-to-LDS buffer loads (written as inline assembly, which the
    compiler's hazard pass does not look into) that read an SGPR a vector
    instruction wrote fewer than `window` wait states earlier: such a load may
    use the SGPR's old value. Returns (line number, load, writer) for each.
    The scan follows the instruction order of the listing and stops at a
    label; s_nop N counts N + 1 wait states."""
    insts = []
    for n, line in enumerate(asm.splitlines(), 1):
        t = line.split(";")[0].strip()
        if not t or (t.startswith(".") and not t.endswith(":")):  # directives; labels are kept
            continue
        insts.append((n, t))
    found = []
    for i, (n, t) in enumerate(insts):
        if not (t.startswith("buffer_load") and t.endswith(" lds")):
            continue
        regs = _sgprs(t.split(None, 1)[1])
        waits = 0
        for j in range(i - 1, -1, -1):
            pt = insts[j][1]
            if pt.endswith(":") or waits >= window:
                break
            if pt.startswith("s_nop"):
                waits += int(pt.split()[1], 0) + 1
                continue
            if pt.startswith("v_"):
                dst = pt.split(None, 1)[1].split(",")[0] if " " in pt else ""
                if _sgprs(dst) & regs:
                    found.append((n, t, pt))
                    break
            waits += 1
    return found


def build(verbose: bool = False, jobs: int | None = None) -> pathlib.Path:
    cc = hipcc()
    BUILD.mkdir(exist_ok=True)
    sources = sorted(CSRC.glob("*.hip"))
    calib = sorted((PKG / "calib").glob("*.hip"))
    objs = [BUILD / (s.stem + ".o") for s in sources]
    calib_objs = [BUILD / ("calib_" + s.stem + ".o") for s in calib]

    def compile_one(pair):
        src, obj = pair
        # -save-temps=obj also leaves the device assembly next to the object
        out = _run([cc, *COMMON_FLAGS, "-save-temps=obj", "-c", str(src), "-o", str(obj)])
        if verbose and out.strip():
            print(out)
        return obj

    jobs = jobs or min(len(sources) + len(calib), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(compile_one, zip(sources + calib, objs + calib_objs)))
    problems = []
    for src in sources + calib:
        for asm_file in BUILD.glob(src.stem + "-hip-amdgcn-amd-amdhsa-*.s"):
            problems += [f"{asm_file.name}:{n}: {load}  <- {writer}"
                         for n, load, writer in vmem_sgpr_hazards(asm_file.read_text())]
    if problems:
        raise RuntimeError("direct-to-LDS loads reading an SGPR written by a vector instruction fewer than 5 wait "
                           "states earlier:\n" + "\n".join(problems[:20]))
    for f in BUILD.iterdir():  # the compiler's intermediate files, scanned above
        if "-hip-amdgcn-" in f.name or "-host-" in f.name or f.name.endswith(".hipfb"):
            f.unlink()
    for lib, lib_objs in ((LIB, objs), (CALIB_LIB, calib_objs)):
        tmp = lib.with_suffix(".so.tmp")
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, lib_objs)])
        os.replace(tmp, lib)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
