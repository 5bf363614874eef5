"""Build libboundary.so in-tree with hipcc for gfx950.

Each translation unit compiles to an object under ``_build/`` (in parallel),
then hipcc links the shared library next to this file. Packed fp32 VALU ops
are switched off for all device code. A second, separate library,
libboundary_ceiling.so, holds the streaming kernel the benchmark uses as a
context figure; it is not part of the boundary library.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libboundary.so")
CEILING_LIB_PATH = os.path.join(HERE, "libboundary_ceiling.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["host.cpp", "k_read.hip", "k_partials.hip", "k_moe.hip", "k_complete.hip", "k_wave.hip",
           "k_wave_complete.hip"]
CEILING_SOURCES = ["ceiling.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIPFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden", "-I", INCLUDE,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = {}
    for src in SOURCES + CEILING_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs[src] = obj
        cmd = [HIPCC, *HIPFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature name; that warning is expected
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(text)
        elif lines and verbose:
            sys.stderr.write("\n".join(lines) + "\n")
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    for path, srcs in ((LIB_PATH, SOURCES), (CEILING_LIB_PATH, CEILING_SOURCES)):
        tmp = path + ".tmp"
        subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
                               *(objs[s] for s in srcs)])
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
