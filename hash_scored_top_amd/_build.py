"""Build libhst.so (all HIP kernels + the C ABI) in-tree for gfx950."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhst.so")
BUILD = os.path.join(PKG, "_build")
# the bounds-checked debug build: HST_DEBUG, relocatable device code (one
# device word of check results shared by every kernel)
LIB_DEBUG = os.path.join(PKG, "libhst_debug.so")
BUILD_DEBUG = os.path.join(PKG, "_build_debug")
DEBUG_FLAGS = ["-DHST_DEBUG", "-fgpu-rdc", "-Wno-pass-failed"]  # (its checks stop some unrolling)

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=on",
    # never let the compiler emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 8, debug: bool = False) -> str:
    """Compile every csrc/*.hip to an object, then link libhst.so (or, with
    debug, the bounds-checked libhst_debug.so)."""
    bdir, lib = (BUILD_DEBUG, LIB_DEBUG) if debug else (BUILD, LIB)
    extra = DEBUG_FLAGS if debug else []
    os.makedirs(bdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    # objects of sources that no longer exist would otherwise linger in the
    # build folder (they are never linked, but they are shipped with the tree)
    live = {os.path.basename(s) + ".o" for s in srcs}
    for stale in glob.glob(os.path.join(bdir, "*.o")):
        if os.path.basename(stale) not in live:
            os.remove(stale)
    objs = []
    procs = []
    for src in srcs:
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
        if len(procs) >= jobs:
            _drain(procs[:1]); procs = procs[1:]
    _drain(procs)
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if out.returncode != 0:
        raise RuntimeError("link failed:\n" + out.stdout)
    os.replace(tmp, lib)
    return lib


def _drain(procs):
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
        warn = [ln for ln in out.splitlines()
                if "warning" in ln and "packed-fp32-ops" not in ln]
        if warn:
            sys.stderr.write(out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--debug" in sys.argv))
