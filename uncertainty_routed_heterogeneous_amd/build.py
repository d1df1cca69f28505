"""Build libhetattn.so (gfx950) in-tree with hipcc.

Usage: ``python -m uncertainty_routed_heterogeneous_amd.build``.  The library
lands next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhetattn.so")
SOURCES = ["api.cpp", "route.hip", "dense.hip", "local.hip", "backward.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU ops stay disabled: plain fp32 code must not be turned into
# v_pk_{add,mul,fma}_f32.  The host pass warns that it does not know the
# feature; that warning is harmless.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-ffp-contract=fast", "-munsafe-fp-atomics"]


def _run(cmd, verbose: bool):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the
    shared library; every call compiles from scratch."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    objs = [os.path.join(objdir, s + ".o") for s in SOURCES]
    cmds = [[HIPCC, *compile_flags, *inc, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", 0)) or (os.cpu_count() or 1)))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    # A kernel whose host-side stub the compiler did not emit leaves an
    # undefined __device_stub__ symbol, which only fails when the library is
    # loaded; refuse such a build here.
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "__device_stub__" in l]
    if nm.returncode != 0 or missing:
        os.remove(tmp)
        raise RuntimeError("kernel stubs missing from the host pass: " + ", ".join(missing or [nm.stderr]))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
