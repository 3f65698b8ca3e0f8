"""The largest list the ABI takes (k = 4096) on a row of 4500 blocks
(288 000 tokens): the two-call path, the fused step and the ordered list
with the early stop, against the oracle.  These go through the selection's
general branches (bisection and radix selects, the entry-by-entry rank of a
long ordered list) and a decode of 4097 items per row."""

from __future__ import annotations

import pytest
import torch

import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = {
    "two-call": (False, 64, False),
    "fused": (False, 64, True),
    "ordered": (True, 0, False),
}


@pytest.mark.parametrize("case", list(CASES))
def test_largest_k(case):
    ordered, k_e, fused = CASES[case]
    cfg = W.Config(f"limits-{case}", 300 + list(CASES).index(case), batch=1,
                   context=64 * 4500 + 7, num_q_heads=4, num_kv_heads=1, head_dim=128,
                   dtype="bf16", mode="group_softmax", k=4096, k_e=k_e, steps=1,
                   ordered=ordered, tau=1e-3 if ordered else 0.0)
    H.run_and_check(cfg, fused=fused)
