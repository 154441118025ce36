"""Build libcsa.so (HIP for gfx950) in-tree with hipcc.

    python sparse_attention_thd_amd/build.py        # or build() from Python (__graft_entry__.build)

Compiles every ``csrc/*.hip`` to an object file in ``_build/`` and links
``sparse_attention_thd_amd/libcsa.so``.  Always recompiles (a full build takes
well under a minute).  ``--debug`` (``build(debug=True)``) also links
``libcsa_debug.so``: the same objects with ``csa_api.hip`` compiled with
``CSA_DEBUG`` defined, whose calls check their index rows (csa_validate_topk_rows)
before launching.  Point ``CSA_LIBRARY`` at it to load it instead of libcsa.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcsa.so")
DEBUG_LIB = os.path.join(PKG, "libcsa_debug.so")
ARCH = os.environ.get("CSA_OFFLOAD_ARCH", "gfx950")

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set HIPCC)")


def _compile(hipcc, src, obj, extra=()):
    cmd = [hipcc, *HIP_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(hipcc, objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, debug: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = [(s, o, ()) for s, o in zip(srcs, objs)]
    api_dbg = os.path.join(BUILD, "csa_api_debug.o")
    if debug:
        jobs.append((os.path.join(CSRC, "csa_api.hip"), api_dbg, ("-DCSA_DEBUG",)))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda j: _compile(hipcc, *j), jobs))
    _link(hipcc, objs, LIB)
    if verbose:
        print(f"built {LIB}")
    if debug:
        _link(hipcc, [api_dbg if o.endswith("csa_api.o") else o for o in objs], DEBUG_LIB)
        if verbose:
            print(f"built {DEBUG_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, debug="--debug" in sys.argv[1:])
    sys.exit(0)
