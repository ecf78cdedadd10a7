"""Compile libssc.so (all HIP sources of the package) for gfx950 with hipcc, in-tree.

Every source is compiled to its own object in parallel (under ``_build/``), then linked.  The
library embeds a digest of its sources (``ssc_source_digest()``), which the binding compares
with the sources on disk before it loads the library, so a stale build is never used.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libssc.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = ["abi.hip", "index.hip", "conv.hip", "resample.hip", "norm.hip", "ablation.hip",
           "gemm.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # Keep the compiler from forming packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def source_files() -> list:
    """Every file the library is built from: the HIP sources and headers of csrc/ and the
    public header, in a fixed order."""
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))
             if f.endswith((".hip", ".h"))]
    files.append(os.path.join(INCLUDE, "ssc.h"))
    return files


def source_digest() -> str:
    """sha256 (first 16 hex digits) over the names and contents of source_files()."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.relpath(path, ROOT).encode())
        h.update(b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def build(verbose: bool = False, jobs: int = 0) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJDIR, exist_ok=True)
    digest = source_digest()
    jobs = jobs or min(len(SOURCES), max(1, min(os.cpu_count() or 1, 8)))

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPCC_FLAGS, "-c", "-I", INCLUDE, "-I", CSRC,
               f"-DSSC_SOURCE_DIGEST=\"{digest}\"", os.path.join(CSRC, src), "-o", obj + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(obj + ".tmp", obj)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
