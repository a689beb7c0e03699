"""Build libfp8q.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: ``python fp8_precision_quant_amd/build.py`` (run as a file: importing
the package would first load the existing library), or ``__graft_entry__.build()``.
Every source is compiled on each call; objects are compiled in parallel and
linked in-tree next to this file, so the library travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8q.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# packed fp32 VALU instructions are disabled for every device compile
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]

SOURCES = ["api.hip", "check.hip", "quant.hip", "quant_transpose.hip", "gemm.hip", "gemm_nk.hip", "gemm_w4.hip", "adam.hip"]


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on %s" % src)


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs,
                           "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
