"""The two-call selection with rows split into several chunks (forced small
with NSA_SELECT_CHUNK), through every branch of the row's last workgroup:
gather-and-rank from registers, the shared-memory fallback for more than 16
query-aware blocks or more than 2048 blocks, and the ordered list sorted by
a bitonic network (up to 256 entries) or ranked entry by entry (more)."""

from __future__ import annotations

import pytest
import torch

import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = {
    # name: (chunk, context, k, k_e, ordered)
    "registers": ("512", 64 * 600 + 9, 24, 8, False),
    "more-than-16": ("512", 64 * 600 + 9, 40, 8, False),
    "more-than-2048-blocks": ("1024", 64 * 2100 + 5, 24, 8, False),
    "ordered-bitonic": ("512", 64 * 600 + 9, 48, 0, True),
    "ordered-ranked": ("512", 64 * 600 + 9, 300, 0, True),
}


@pytest.mark.parametrize("case", list(CASES))
def test_select_chunks(case, monkeypatch):
    chunk, context, k, k_e, ordered = CASES[case]
    monkeypatch.setenv("NSA_SELECT_CHUNK", chunk)
    cfg = W.Config(f"chunks-{case}", 95 + list(CASES).index(case), batch=2, context=context,
                   num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16",
                   mode="group_softmax", k=k, k_e=k_e, steps=2, ordered=ordered,
                   tau=1e-3 if ordered else 0.0)
    H.run_and_check(cfg)
