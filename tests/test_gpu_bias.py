"""The ED-DMA attention-bias variant (nsa_sparse_decode_biased) against the
oracle: the eviction logit of every token added to its attention logit
(NOSA summary, "ED-DMA"), on the plain split-K decode and on the early-stop
walk, whose masses take the same logits.  Selection is unchanged (it scores
pre-exponential eviction scores), so the oracle attends the GPU's list."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import nsa_oracle as O
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _run(cfg, steps):
    batch = W.build_batch(cfg)
    layer = H.make_layer(cfg, batch)
    H.prefill(layer, cfg)
    dev = layer.device
    for t in range(steps):
        L = cfg.seq_len(t)
        lens = np.full(cfg.batch, L, dtype=np.int32)
        layer.seq_lens.copy_(torch.from_numpy(lens))
        if L % 64 == 0:
            first = torch.full((cfg.batch,), L // 64 - 1, dtype=torch.int32, device=dev)
            layer.update_reps(first, torch.ones(cfg.batch, dtype=torch.int32, device=dev), 1)
        layer.select(H.device_query(cfg, t), L)
        layer.decode(H.device_q(cfg, t), bias=layer.evict_logits)
        res = H.fetch(layer)
        yield t, L, res


def _check_rows(cfg, t, L, res, n_star_stats):
    G = cfg.group
    for b in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            ri = W.row_inputs(cfg, b, g)
            keys = W.stored_to_f64(ri.keys, cfg.dtype)
            values = W.stored_to_f64(ri.values, cfg.dtype)
            bias = ri.logits.astype(np.float64)
            q = W.stored_to_f64(W.query_row(cfg, b, g, t), cfg.dtype)
            scale = 1.0 / math.sqrt(cfg.head_dim)
            n = int(res.num_selected[b, g])
            sel = [int(x) for x in res.selected[b, g, :n]]
            if cfg.ordered:
                n_gpu = int(res.num_processed[b, g])
                n_ora, _ = O.early_stop_attention(q, keys, values, sel, L, cfg.tau, scale, bias)
                assert abs(n_gpu - n_ora) <= 1, (b, g, n_gpu, n_ora)
                n_star_stats.append((n_gpu, n_ora))
                sel = sel[:n_gpu]
            want = O.sparse_attention(q, keys, values, sel, L, scale, bias)
            got = res.out[b, g * G:(g + 1) * G]
            err = np.abs(got - want).max()
            assert err <= H.TOL[cfg.dtype], (b, g, t, err)
            plain = O.sparse_attention(q, keys, values, sel, L, scale)
            assert np.abs(want - plain).max() > 2 * H.TOL[cfg.dtype], "bias had no effect"


@pytest.mark.parametrize("dtype,D,G", [("bf16", 128, 4), ("f32", 64, 2), ("bf16", 128, 8)])
def test_biased_decode_matches_oracle(dtype, D, G):
    cfg = W.Config(f"bias-{dtype}-{D}-{G}", 90, batch=3, context=64 * 41 + 37, num_q_heads=2 * G,
                   num_kv_heads=2, head_dim=D, dtype=dtype, mode="group_softmax", k=12, k_e=8,
                   steps=30)
    H.log(f"[case] biased decode {dtype} D={D} G={G}")
    for t, L, res in _run(cfg, 28):
        if t in (0, 26, 27):        # step 26 fills a block
            _check_rows(cfg, t, L, res, [])


def test_biased_early_stop_matches_oracle():
    cfg = W.Config("bias-es", 91, batch=2, context=64 * 120 + 9, num_q_heads=8, num_kv_heads=2,
                   head_dim=128, dtype="bf16", mode="group_softmax", k=48, k_e=0, steps=2,
                   ordered=True, tau=1e-3, planted_scale=16.0)
    H.log("[case] biased early-stop walk")
    stats = []
    for t, L, res in _run(cfg, 2):
        _check_rows(cfg, t, L, res, stats)
    exact = sum(1 for a, b in stats if a == b)
    assert exact >= len(stats) - 1, stats
