"""Build libattn_mi355x.so in-tree for gfx950.

    python -m exact_masked_scaled_amd.build [--jobs N] [--verbose]

HIP kernel sources are compiled with hipcc for gfx950 only; the host-side
validation and dispatch (plain C++) with g++.  Objects go to
exact_masked_scaled_amd/_build/, the library next to this file.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattn_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
ROCM_LIB = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
LINK_LIBS = ["-L", ROCM_LIB, "-lrocblas", f"-Wl,-rpath,{ROCM_LIB}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout or "") + (res.stderr or "")
    # hipcc's host pass does not know the packed-fp32 feature name; harmless
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source (always, even if a library exists) and link."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    hip, cpp = sources()
    cmds = []
    objs = []
    for f in hip:
        o = os.path.join(BUILD, f + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    cxx = os.environ.get("CXX", "g++")
    for f in cpp:
        o = os.path.join(BUILD, f + ".o")
        cmds.append([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    jobs = jobs or min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    # the projections' products link the vendor GEMM
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs, *LINK_LIBS], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    path = build(a.jobs, a.verbose)
    print(path)


if __name__ == "__main__":
    sys.exit(main())
