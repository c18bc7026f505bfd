"""Build the gfx950 HIP library in-tree with hipcc.

The library is one shared object, ``libsla.so``, next to this file; its C ABI
is declared in ``include/sla.h`` at the repository root.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsla.so")
LIB_DEBUG = os.path.join(PKG, "libsla_debug.so")
SOURCES = ["setup.hip", "solver.hip", "multi.hip", "noalloc.hip", "host_util.cpp", "spectrum.cpp",
           "trace.cpp", "api.cpp"]
ARCH = os.environ.get("SLA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            # never emit packed fp32 arithmetic (see the design notes)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wextra", "-Wno-unused-function"]


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every source to an object, then link libsla.so (always rebuilds).
    debug=True builds libsla_debug.so with SLA_DEBUG defined: every gathered
    column index is checked against the vector length on the device, and a
    solve that saw one out of range returns SLA_ERR_INVALID_ARG."""
    objdir = os.path.join(PKG, "_build_debug" if debug else "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc(), *flags(), *(["-DSLA_DEBUG=1"] if debug else []), *lang, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(f"--- {s}\n{o}" for s, o in failed))
    out = LIB_DEBUG if debug else LIB
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-ldl"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--debug" in sys.argv))
