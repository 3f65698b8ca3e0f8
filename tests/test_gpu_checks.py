"""The library built with the device-side contract checks (-DNSA_DEBUG):
each broken item of the caller's contract is recorded with its bit, and a
clean step records nothing.  Runs tests/checks_case.py in a child process
against block_sparse_kv_nsa_amd/libnsa_checks.so."""

from __future__ import annotations

import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_sparse_kv_nsa_amd", "libnsa_checks.so")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.skipif(not os.path.exists(LIB), reason="libnsa_checks.so not built "
                    "(python block_sparse_kv_nsa_amd/build.py --checks)")
def test_contract_violations_are_recorded():
    print("[case] device checks: child process on libnsa_checks.so", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "checks_case.py")],
                       capture_output=True, text=True, cwd=ROOT, timeout=240,
                       env=dict(os.environ, NSA_LIB_PATH=LIB))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    res = {}
    for line in r.stdout.splitlines():
        if line.startswith("RESULT "):
            k, v = line[len("RESULT "):].rsplit(":", 1)
            res[k] = int(v)
    assert res["clean two calls"] == 0 and res["clean fused"] == 0, res
    assert res["table entry two calls"] & 1 and res["table entry fused"] & 1, res
    assert res["listed id"] & 2, res
    assert res["eviction id fused"] & 4, res
    assert res["seq_len"] & 8, res
