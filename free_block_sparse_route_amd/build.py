"""Build libsparse_attn.so in-tree with hipcc for gfx950.

    python free_block_sparse_route_amd/build.py [--verbose]

(run by path: importing the package itself needs the built library)

Each HIP source is compiled to an object under _build/ (in parallel), then
linked into free_block_sparse_route_amd/libsparse_attn.so.  Every call
recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsparse_attn.so")
SOURCES = ("sa_api.hip", "sa_route.hip", "sa_flash.hip", "sa_permute.hip", "sa_sparsepr.hip")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep packed-fp32 VALU instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    return os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err)


def build(verbose: bool = False, extra_flags: list | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    flags = FLAGS + list(extra_flags or [])
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        for src in SOURCES:
            obj = os.path.join(BUILD, src.replace(".hip", ".o"))
            objs.append(obj)
            jobs.append(ex.submit(_run, [cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj], verbose))
        for j in jobs:
            j.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
