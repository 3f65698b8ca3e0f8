"""nsa_decode_step_noalloc (the fused step on the library's own per-device
workspace) against nsa_decode_step with a caller workspace: two calls in a
row, the second with a smaller input; selections, eviction state and outputs
must agree exactly (same kernels, same inputs), and both must pass the oracle
checks.

Every case prints what it runs before touching the GPU.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def one_step_both(cfg: W.Config):
    """Two layers on the same inputs: step 0 through each entry point."""
    H.log(f"[case] no-alloc vs workspace step: {cfg.name} B={cfg.batch} ctx={cfg.context} "
          f"Hq={cfg.num_q_heads} Hkv={cfg.num_kv_heads} D={cfg.head_dim} {cfg.dtype}")
    batch = W.build_batch(cfg)
    ref = H.make_layer(cfg, batch)
    new = H.make_layer(cfg, batch)
    for lay in (ref, new):
        H.prefill(lay, cfg)
    L = cfg.seq_len(0)
    lens = torch.full((cfg.batch,), L, dtype=torch.int32, device="cuda")
    ref.seq_lens.copy_(lens)
    new.seq_lens.copy_(lens)
    query, q = H.device_query(cfg, 0), H.device_q(cfg, 0)
    status = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    ref.step(query, q, L)
    new.step_noalloc(query, q, L, step_status=status)
    torch.cuda.synchronize()
    ref.check_step()
    assert int(status.item()) == 0, "a wait of the no-alloc step expired"
    a, b = H.fetch(ref), H.fetch(new)
    assert np.array_equal(a.selected, b.selected)
    assert np.array_equal(a.num_selected, b.num_selected)
    assert np.array_equal(a.evict_set, b.evict_set)
    assert torch.equal(ref.evict_seen, new.evict_seen)
    err = np.abs(a.out - b.out).max()
    assert err <= H.TOL[cfg.dtype], err
    # and the no-alloc result passes the oracle checks on sampled rows
    for r in H.sample_rows(cfg, 3):
        orow = H.oracle_row(cfg, *r)
        H.check_step(cfg, b, orow, r[0], r[1], 0)
    return err


def test_noalloc_matches_workspace_step_twice_second_smaller():
    big = W.config(1, batch=4, steps=1)
    small = W.config(0)
    e1 = one_step_both(big)
    e2 = one_step_both(small)
    H.log(f"[info] max |out difference| {e1} then {e2}")
