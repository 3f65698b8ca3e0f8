"""Every built kernel instance against the oracle: element type x head_dim x
group size, on the fused step, the two-call path and the early-stop walk,
with a ragged tail and a block filling during the steps."""

from __future__ import annotations

import itertools

import pytest
import torch

import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SHAPES = list(itertools.product(["f32", "bf16"], [64, 128], [1, 2, 4, 8]))
PATHS = ["fused", "split", "early-stop"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype,D,G", SHAPES)
def test_instance(dtype, D, G, path):
    ordered = path == "early-stop"
    cfg = W.Config(f"matrix-{dtype}-{D}-{G}-{path}", 200 + 3 * SHAPES.index((dtype, D, G)) +
                   PATHS.index(path), batch=2, context=64 * 23 + 61, num_q_heads=2 * G,
                   num_kv_heads=2, head_dim=D, dtype=dtype, mode="group_softmax",
                   k=20 if ordered else 10, k_e=0 if ordered else 6, steps=5, ordered=ordered,
                   tau=1e-3 if ordered else 0.0)
    H.run_and_check(cfg, fused=path == "fused")
