"""Build libdas.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree, and
its debug build libdas_debug.so (DAS_DEBUG_LDS_POISON=1: every LDS buffer is
filled with NaN bytes when it stops being live), compiled side by side."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdas.so")
DEBUG_LIB = os.path.join(HERE, "libdas_debug.so")
SOURCES = [os.path.join(CSRC, "das_kernels.hip"), os.path.join(CSRC, "das_api.cpp"),
           os.path.join(CSRC, "das_noalloc.hip")]
HEADERS = [os.path.join(ROOT, "include", "das.h"), os.path.join(CSRC, "das_internal.h")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def command(out: str = LIB, debug: bool = False) -> list:
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 (v_pk_*_f32) stays off: plain fp32 VALU code only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            *(["-DDAS_DEBUG_LDS_POISON=1"] if debug else []),
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *SOURCES, "-o", out]


def build(verbose: bool = False) -> str:
    """Compile both libraries (two hipcc processes at once); returns LIB."""
    jobs = []
    for lib, debug in ((LIB, False), (DEBUG_LIB, True)):
        cmd = command(lib + ".tmp", debug)
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((lib, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                           text=True)))
    failed = []
    for lib, proc in jobs:
        out, err = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(out + err)
            failed.append(os.path.basename(lib))
    if failed:
        raise RuntimeError("hipcc failed building " + ", ".join(failed))
    for lib, _ in jobs:
        os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
