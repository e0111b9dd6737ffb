"""Builds libspmv_amd.so (HIP kernels + C ABI) for gfx950 with hipcc.

Usage: python -m sparse_matrix_vector_amd.csrc.build   (or build() from Python)

Every source file under this directory is compiled to an object in
``sparse_matrix_vector_amd/_build`` and linked into
``sparse_matrix_vector_amd/libspmv_amd.so``.  Packed fp32 instructions are
disabled (``-packed-fp32-ops``); float atomics use the hardware instruction
(``-munsafe-fp-atomics``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libspmv_amd.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", HERE,
]


def sources() -> list[str]:
    return sorted(os.path.join(HERE, f) for f in os.listdir(HERE)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if "warning" in warn:
        sys.stderr.write(warn + "\n")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compiles every source (always) and links the shared library."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
