"""Build libwgn.so (HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libwgn.so")
SOURCES = [os.path.join(CSRC, f) for f in ("wgn_kernels.hip", "wgn_attn.hip", "wgn_int4.hip", "wgn_read.hip", "wgn_gemm.hip", "wgn_bwd.hip", "wgn_api.cpp")]
HEADERS = [os.path.join(CSRC, f) for f in ("wgn_prog.h", "wgn_loader.h", "wgn_attn.h", "wgn_numerics.h", "wgn_gemm.h", "wgn_bwd.h")] + [os.path.join(INCLUDE, "wgn.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         # packed FP32 ops stay off: plain float code only
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE,
         # per-kernel register/scratch report, checked below
         "-Rpass-analysis=kernel-resource-usage"]


def kernel_resources(report: str):
    """{kernel: {"VGPRs": n, "ScratchSize": n, ...}} from the compiler's
    resource-usage remarks."""
    out, cur = {}, None
    for line in report.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[bytes/lane\])?: (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return out


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile libwgn.so.  `defines` (e.g. ["WGN_DEPTH=8"]) override the
    kernel's tuning constants for experimental builds written to `out`.
    Each source is compiled on its own (in parallel), then linked."""
    tmp = out + ".tmp%d" % os.getpid()
    objs, procs = [], []
    for src in SOURCES:
        obj = "%s.%s.o" % (tmp, os.path.splitext(os.path.basename(src))[0])
        cmd = [HIPCC] + FLAGS + ["-D" + d for d in defines] + ["-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        objs.append(obj)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    report, failed = "", False
    for p in procs:
        so, se = p.communicate()
        report += se
        if p.returncode != 0:
            sys.stderr.write(so + se)
            failed = True
    try:
        if failed:
            raise RuntimeError("hipcc failed building libwgn.so")
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        if verbose:
            print(" ".join(link), flush=True)
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed linking libwgn.so")
    finally:
        for o in objs:
            if os.path.exists(o):
                os.unlink(o)
    # The streaming kernels must keep everything in registers and LDS: a
    # spill to scratch memory puts global-memory latency on the hot path.
    res = kernel_resources(report)
    spills = {k: v.get("ScratchSize") for k, v in res.items() if v.get("ScratchSize", 0) > 0}
    if not res or spills:
        os.unlink(tmp)
        raise RuntimeError("libwgn.so kernels use scratch memory: %r" % (spills or "no resource report"))
    with open(out + ".resources.txt", "w") as f:
        for k in sorted(res):
            f.write("%s %s\n" % (k, " ".join("%s=%d" % kv for kv in sorted(res[k].items()))))
    os.replace(tmp, out)
    return out


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
