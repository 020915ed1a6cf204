"""Build libsta.so (HIP kernels for gfx950 + the C-ABI layer) in-tree.

    python -m sparse_attention_video_tile_amd.build [--verbose]

HIP sources are compiled with hipcc for gfx950 only; the C-ABI layer is plain
C++ compiled with g++. Packed fp32 instructions are disabled for device code.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsta.so")
# The same library with the attention kernels built single-buffered (one K/V
# buffer, loads after every wave has finished a chunk): the reference of the
# synchronisation audit test. Built beside libsta.so, never loaded by the
# package itself.
AUDIT_LIB = os.path.join(PKG, "libsta_audit.so")
AUDIT_FLAGS = ["-DSTA_AUDIT_SINGLE_BUFFER=1"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_SOURCES = ["sta_layout.hip", "sta_attention.hip", "sta_backward.hip", "sta_recall.hip",
               "sta_scratch.hip"]
CXX_SOURCES = ["sta_api.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast",
    "-fno-honor-nans",
    "-Wno-unused-command-line-argument",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def _hipcc() -> str:
    return shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(
        line for line in r.stdout.splitlines()
        if "packed-fp32-ops' is not a recognized feature" not in line
    )
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, extra_hip_flags=()) -> str:
    """Compile every source and link libsta.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([_hipcc(), *HIPCC_FLAGS, *extra_hip_flags, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append(["g++", *CXX_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
    audit_obj = os.path.join(BUILD, "sta_attention_audit.hip.o")
    jobs.append([_hipcc(), *HIPCC_FLAGS, *extra_hip_flags, *AUDIT_FLAGS, *inc, "-c",
                 os.path.join(CSRC, "sta_attention.hip"), "-o", audit_obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    for lib, lib_objs in ((LIB, objs),
                          (AUDIT_LIB, [audit_obj if o.endswith("sta_attention.hip.o") else o for o in objs])):
        tmp = lib + ".tmp"
        _run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *lib_objs, "-o", tmp], verbose)
        os.replace(tmp, lib)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(verbose=args.verbose)
    print(path)


if __name__ == "__main__":
    sys.exit(main())
