"""Build libnsa.so for gfx950 with hipcc (in-tree, next to this file).

    python block_sparse_kv_nsa_amd/build.py [--debug]

(run by path: importing the package itself loads the library being built)

Every HIP source is compiled for gfx950 only; packed-fp32 instructions are
turned off (-packed-fp32-ops).  Objects go to _build/ at the repository
root; the shared library lands in the package directory.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnsa.so")

SOURCES = ["nsa_api.cpp", "nsa_reps.hip", "nsa_select.hip", "nsa_decode.hip", "nsa_step.hip",
           "nsa_residency.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnsa)")


def common_flags(debug: bool) -> list[str]:
    flags = ["-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]
    flags += ["-O1", "-g"] if debug else ["-O3"]
    return flags


def compile_one(src: str, debug: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc()] + common_flags(debug)
    if src.endswith(".hip"):
        cmd += ["-x", "hip", f"--offload-arch={ARCH}",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-fno-gpu-rdc", "-mcode-object-version=5"]
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(debug: bool = False, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: compile_one(s, debug), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5",
           "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--debug", action="store_true")
    args = ap.parse_args(argv)
    build(debug=args.debug)
    return 0


if __name__ == "__main__":
    sys.exit(main())
