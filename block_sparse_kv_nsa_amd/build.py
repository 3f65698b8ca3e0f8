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
LIB_CHECKS = os.path.join(PKG, "libnsa_checks.so")

SOURCES = ["nsa_api.cpp", "nsa_reps.hip", "nsa_select.hip", "nsa_decode.hip", "nsa_step.hip",
           "nsa_residency.hip", "nsa_prefill.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnsa)")


def common_flags(debug: bool, checks: bool = False) -> list[str]:
    flags = ["-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]
    flags += ["-O1", "-g"] if debug else ["-O3"]
    if checks:
        flags += ["-DNSA_DEBUG"]
    return flags


def compile_one(src: str, debug: bool, checks: bool = False) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, ("checks_" if checks else "") + src + ".o")
    cmd = [hipcc()] + common_flags(debug, checks)
    if src.endswith(".hip"):
        cmd += ["-x", "hip", f"--offload-arch={ARCH}",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-fno-gpu-rdc", "-mcode-object-version=5"]
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(debug: bool = False, verbose: bool = True, checks: bool = False) -> str:
    """Compile every source for gfx950 and link the library: libnsa.so, or
    with checks=True libnsa_checks.so (the device-side contract checks,
    -DNSA_DEBUG)."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: compile_one(s, debug, checks), SOURCES))
    lib_path = LIB_CHECKS if checks else LIB
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5",
           "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


def build_asan(verbose: bool = True) -> str:
    """A copy of the library whose host code (the C-ABI layer, nsa_api.cpp)
    is built with AddressSanitizer by the host compiler, linked with the
    release kernels' objects from _build/ (run build() first).  For CPU
    tests of the argument checks; load it with libasan preloaded."""
    out_dir = os.path.join(BUILD, "asan")
    os.makedirs(out_dir, exist_ok=True)
    api_obj = os.path.join(out_dir, "nsa_api_asan.o")
    lib = os.path.join(out_dir, "libnsa_asan.so")
    gxx = shutil.which("g++") or "g++"
    cmd = [gxx, "-std=c++17", "-fPIC", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "nsa_api.cpp"), "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"asan compile failed: {' '.join(cmd)}\n{r.stderr}")
    objs = [os.path.join(BUILD, s + ".o") for s in SOURCES if s.endswith(".hip")]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"kernel objects missing (run build() first): {missing}")
    cmd = [gxx, "-shared", "-fsanitize=address", "-o", lib, api_obj] + objs + [
        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"asan link failed: {' '.join(cmd)}\n{r.stderr}")
    if verbose:
        print(f"built {lib}")
    return lib


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("--checks", action="store_true",
                    help="also build libnsa_checks.so (device-side contract checks, -DNSA_DEBUG)")
    ap.add_argument("--asan", action="store_true",
                    help="also build _build/asan/libnsa_asan.so (host code under AddressSanitizer)")
    args = ap.parse_args(argv)
    build(debug=args.debug)
    if args.checks:
        build(debug=args.debug, checks=True)
    if args.asan:
        build_asan()
    return 0


if __name__ == "__main__":
    sys.exit(main())
