"""Compile the gfx950 HIP sources into libpagedattn.so (in the package
directory).  Runs on a machine without a GPU: hipcc cross-compiles."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpagedattn.so")
# the trace library: the same sources with the timeline trace points compiled
# in (pa_trace_set; PA_TRACE=1 makes the package load it)
TRACE_LIB = os.path.join(HERE, "libpagedattn_trace.so")
ARCH = "gfx950"
SOURCES = ["api.hip", "reshape_and_cache.hip", "merge.hip", "decode.hip", "prefill.hip",
           "check.hip", "cascade.hip", "local.hip", "probe.hip", "noalloc.hip"]
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # never let the compiler form packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# Per-source additions.  The prefill kernel assumes no NaN among its inputs:
# its row maxima then compile to plain v_max3 chains, without the operand
# quieting IEEE maxNum otherwise needs (a NaN input gives a NaN-or-garbage
# result either way).
EXTRA = {"prefill.hip": ["-fno-honor-nans"]}


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False, trace: bool = False) -> str:
    out_dir = BUILD + ("_trace" if trace else "")
    lib_path = TRACE_LIB if trace else LIB
    os.makedirs(out_dir, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *FLAGS, *EXTRA.get(src, []), *(["-DPA_TRACE=1"] if trace else []),
                     "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        for r in ex.map(_run, cmds):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout + r.stderr, file=sys.stderr)
    tmp = lib_path + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True, trace="--trace" in sys.argv[1:]))
