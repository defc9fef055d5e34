"""Build libwgn.so (HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libwgn.so")
SOURCES = [os.path.join(CSRC, "wgn_kernels.hip"), os.path.join(CSRC, "wgn_api.cpp")]
HEADERS = [os.path.join(CSRC, f) for f in ("wgn_prog.h", "wgn_loader.h")] + [os.path.join(INCLUDE, "wgn.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         # packed FP32 ops stay off: plain float code only
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile libwgn.so.  `defines` (e.g. ["WGN_DEPTH=8"]) override the
    kernel's tuning constants for experimental builds written to `out`."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-D" + d for d in defines] + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libwgn.so")
    os.replace(tmp, out)
    return out


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
