"""The C-ABI layer's argument checks under AddressSanitizer (CPU only).

nsa_api.cpp is rebuilt by the host compiler with -fsanitize=address and
linked with the release kernel objects; tests/test_abi.py then runs in a
child process against that library with libasan preloaded.  Any invalid
read or write in the checks (or their error messages) aborts the child with
a report.
"""

from __future__ import annotations

import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD_PY = os.path.join(ROOT, "block_sparse_kv_nsa_amd", "build.py")


def _build_module():
    spec = importlib.util.spec_from_file_location("nsa_build_asan", BUILD_PY)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs the host compiler")
def test_abi_checks_under_address_sanitizer():
    mod = _build_module()
    objs = [os.path.join(mod.BUILD, s + ".o") for s in mod.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects not built (python block_sparse_kv_nsa_amd/build.py)")
    lib = mod.build_asan(verbose=False)
    asan_rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    env = dict(os.environ, NSA_LIB_PATH=lib, LD_PRELOAD=asan_rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, cwd=ROOT, env=env, timeout=600)
    assert r.returncode == 0 and "AddressSanitizer" not in r.stderr, (
        r.stdout[-3000:] + r.stderr[-3000:])
