"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Acceptance rules are in tests/gpu_harness.py.  Every test prints the case it
is about to run (config, shape, step) before touching the GPU.
"""

from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import nsa_oracle as O
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


# ----------------------------------------------------------------------------
# the five workloads at their own sizes
# ----------------------------------------------------------------------------
def test_config0_tiny_fp32():
    H.run_and_check(W.config(0))


def test_config1_nosa_1b_all_rows():
    _, st = H.run_and_check(W.config(1))
    assert st["gamma_min"] >= 0.75


def test_config1_fill_steps():
    """160 steps: blocks 256 and 257 fill at steps 63 and 127 (incremental
    reps, eviction merges, gamma at fill steps)."""
    cfg = W.config(1, steps=160, batch=4)
    _, st = H.run_and_check(cfg, check_every=3)
    assert st["gamma_min"] >= 0.75


def test_config2_sparda_sampled_rows():
    cfg = W.config(2)
    H.run_and_check(cfg, rows=H.sample_rows(cfg, 12))


def test_config2_sparda_inference_window_sampled_rows():
    """The sparda-8b workload scored on the (32, 16) inference window."""
    cfg = W.config(2).replace(name="sparda-8b-window", mode="forecast_window")
    H.run_and_check(cfg, rows=H.sample_rows(cfg, 12))


def test_config3_long_context_sampled_rows():
    cfg = W.config(3)
    _, st = H.run_and_check(cfg, rows=H.sample_rows(cfg, 6), check_every=3)
    assert st["gamma_min"] >= 0.75


def test_config3_fill_steps():
    """Config 3 for 80 steps: block 2048 fills at step 63 (incremental reps
    and eviction scores at nb = 2049, the eviction merge over a 2049-block
    row, gamma at the fill step)."""
    cfg = W.config(3, steps=80)
    _, st = H.run_and_check(cfg, rows=H.sample_rows(cfg, 4), check_every=8)
    assert st["gamma_min"] >= 0.75


_C4 = {}


def config4_batch():
    """Full-size config-4 pools, built once per session (17 GB of bf16)."""
    if not _C4:
        cfg = W.config(4)
        sample = H.sample_rows(cfg, 6)
        H.log("[case] building config4 pools (sampled rows replicated)")
        _C4["v"] = (cfg, sample) + H.replicated_batch(cfg, sample)
    return _C4["v"]


def test_config4_early_stop_sampled_rows():
    cfg, sample, batch, ris = config4_batch()
    layer, st = H.run_and_check(cfg, rows=sample, batch=batch, row_inputs=ris)
    H.log(f"[info] config4 n* = {st['n_star']}")
    del layer
    torch.cuda.empty_cache()


def test_config4_dense_reference():
    """k = all blocks, no scoring: the decode over every block equals dense
    attention (sampled rows)."""
    cfg, sample, batch, ris = config4_batch()
    H.log(f"[case] config4 dense: all {cfg.nb0} blocks")
    layer = H.make_layer(cfg, batch)
    L = cfg.seq_len(0)
    nb = L // 64
    layer.seq_lens.fill_(L)
    sel = torch.arange(nb, dtype=torch.int32, device="cuda").repeat(cfg.batch, cfg.num_kv_heads, 1)
    nsel = torch.full((cfg.batch, cfg.num_kv_heads), nb, dtype=torch.int32, device="cuda")
    layer.decode(H.device_q(cfg, 0), selected=sel.contiguous(), num_selected=nsel,
                 max_selected=nb, early_stop=False)
    out = H.to_f64(layer.out)
    for (b, g) in sample:
        orow = H.oracle_row(cfg, b, g, ri=ris[(b, g)])
        q = W.stored_to_f64(W.query_row(cfg, b, g, 0), cfg.dtype)
        want = O.dense_attention(q, orow.keys, orow.values, L, orow.scale)
        G = cfg.group
        err = np.abs(out[b, g * G:(g + 1) * G] - want).max()
        assert err <= H.TOL[cfg.dtype], err


# ----------------------------------------------------------------------------
# every built (dtype, head_dim, group, mode) on small ragged shapes
# ----------------------------------------------------------------------------
SMALL = [
    ("f32", 64, 1, "group_softmax", False),
    ("f32", 128, 2, "group_softmax", False),
    ("bf16", 64, 8, "group_softmax", False),
    ("bf16", 128, 4, "group_softmax", False),
    ("bf16", 128, 4, "forecast", False),
    ("f32", 64, 4, "forecast", False),
    ("bf16", 128, 4, "forecast_window", False),
    ("f32", 64, 2, "forecast_window", False),
    ("bf16", 128, 4, "forecast_window", True),
    ("bf16", 128, 8, "group_softmax", True),
    ("f32", 64, 2, "group_softmax", True),
    ("bf16", 64, 1, "group_softmax", True),
]


@pytest.mark.parametrize("dtype,D,G,mode,ordered", SMALL)
def test_small_shapes(dtype, D, G, mode, ordered):
    cfg = W.Config(f"small-{dtype}-{D}-{G}-{mode}-{int(ordered)}", 10 + SMALL.index(
        (dtype, D, G, mode, ordered)), batch=3, context=64 * 41 + 37, num_q_heads=2 * G,
        num_kv_heads=2, head_dim=D, dtype=dtype, mode=mode, k=12 if not ordered else 20,
        k_e=0 if (mode.startswith("forecast") or ordered) else 8, steps=30, ordered=ordered,
        tau=1e-3 if ordered else 0.0)
    H.run_and_check(cfg)


def test_peaked_early_stop_triggers():
    """Planted keys 16u make attention peaked: the stop must fire before the
    cap (at 8u the planted mass is too small for tau = 1e-3 at this shape)."""
    cfg = W.Config("peaked", 30, batch=2, context=64 * 300, num_q_heads=8, num_kv_heads=2,
                   head_dim=128, dtype="bf16", mode="group_softmax", k=64, k_e=0, steps=2,
                   ordered=True, tau=1e-3, planted_scale=16.0)
    _, st = H.run_and_check(cfg)
    assert min(st["n_star"]) < cfg.k, st["n_star"]


# ----------------------------------------------------------------------------
# invariances, determinism, state
# ----------------------------------------------------------------------------
def small_cfg(**kw):
    base = dict(batch=2, context=64 * 50 + 11, num_q_heads=8, num_kv_heads=2, head_dim=128,
                dtype="bf16", mode="group_softmax", k=16, k_e=12, steps=4)
    base.update(kw)
    return W.Config("inv", 40, **base)


def test_block_table_permutation_invariance():
    a = small_cfg(permuted_table=False)
    b = small_cfg(permuted_table=True)
    H.log("[case] identity vs permuted block table")
    outs = []
    for cfg in (a, b):
        layer = H.make_layer(cfg, W.build_batch(cfg))
        H.prefill(layer, cfg)
        for t in range(cfg.steps):
            H.run_step(layer, cfg, t)
        outs.append(H.fetch(layer))
    assert np.array_equal(outs[0].selected, outs[1].selected)
    assert np.array_equal(outs[0].out, outs[1].out)


def test_split_count_invariance(monkeypatch):
    cfg = small_cfg(steps=1)
    batch = W.build_batch(cfg)
    outs = []
    for bpw in ("1", "3", "8"):
        H.log(f"[case] decode blocks per split = {bpw}")
        monkeypatch.setenv("NSA_DECODE_BPW", bpw)
        layer = H.make_layer(cfg, batch)
        H.prefill(layer, cfg)
        H.run_step(layer, cfg, 0)
        outs.append(H.fetch(layer))
    for o in outs[1:]:
        assert np.array_equal(o.selected, outs[0].selected)
        assert np.abs(o.out - outs[0].out).max() <= 1e-2  # one bf16 rounding apart at most


def test_determinism_and_counter_reset():
    cfg = small_cfg(steps=1)
    batch = W.build_batch(cfg)
    H.log("[case] determinism")
    res = []
    for rep in range(3):
        layer = H.make_layer(cfg, batch)
        H.prefill(layer, cfg)
        H.run_step(layer, cfg, 0)
        H.run_step(layer, cfg, 0)  # same step again on the same buffers
        res.append(H.fetch(layer))
        torch.cuda.synchronize()
        rows = cfg.rows
        assert int(layer.sel_ws[: 4 * rows].view(torch.int32).abs().sum()) == 0
        assert int(layer.dec_ws[: 4 * rows].view(torch.int32).abs().sum()) == 0
    for r in res[1:]:
        assert np.array_equal(r.selected, res[0].selected)
        assert np.array_equal(r.out, res[0].out)


def test_checkpoint_resume():
    """The state that crosses steps is the reps, E and the eviction state:
    copying them and resuming matches an uninterrupted run bit for bit."""
    cfg = small_cfg(steps=40, context=64 * 50 + 3)
    batch = W.build_batch(cfg)
    H.log("[case] checkpoint / resume")
    full = H.make_layer(cfg, batch)
    H.prefill(full, cfg)
    snap = None
    for t in range(cfg.steps):
        if t == 20:
            torch.cuda.synchronize()
            snap = {k: getattr(full, k).clone() for k in ("reps", "evict_scores", "evict_set",
                                                            "evict_seen")}
        H.run_step(full, cfg, t)
    want = H.fetch(full)
    resumed = H.make_layer(cfg, batch)
    for k, v in snap.items():
        getattr(resumed, k).copy_(v)
    for t in range(20, cfg.steps):
        H.run_step(resumed, cfg, t)
    got = H.fetch(resumed)
    assert np.array_equal(got.selected, want.selected)
    assert np.array_equal(got.evict_set, want.evict_set)
    assert np.array_equal(got.out, want.out)


def test_bulk_and_incremental_reps_agree():
    cfg = small_cfg()
    batch = W.build_batch(cfg)
    H.log("[case] bulk vs one-block-at-a-time reps")
    a = H.make_layer(cfg, batch)
    H.prefill(a, cfg)
    b = H.make_layer(cfg, batch)
    for blk in range(cfg.nb0):
        first = torch.full((cfg.batch,), blk, dtype=torch.int32, device="cuda")
        one = torch.ones(cfg.batch, dtype=torch.int32, device="cuda")
        b.update_reps(first, one, 1)
    torch.cuda.synchronize()
    assert torch.equal(a.reps, b.reps)
    assert torch.equal(a.evict_scores, b.evict_scores)


# ----------------------------------------------------------------------------
# edge cases: ragged batch, no full block, no tail, nb < k, k_e = k
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("k,k_e", [(8, 4), (8, 8), (8, 0)])
def test_ragged_batch_edges(k, k_e):
    cfg = W.Config("ragged", 50, batch=5, context=64 * 24, num_q_heads=8, num_kv_heads=2,
                   head_dim=128, dtype="bf16", mode="group_softmax", k=k, k_e=k_e, steps=1)
    lens = np.array([37, 64, 64 * 5 + 1, 64 * 20, 64 * 3], dtype=np.int32)
    H.log(f"[case] ragged seq_lens {lens.tolist()} k={k} k_e={k_e}")
    batch = W.build_batch(cfg)
    layer = H.make_layer(cfg, batch)
    first = torch.zeros(cfg.batch, dtype=torch.int32, device="cuda")
    num = torch.from_numpy(lens // 64).to("cuda")
    layer.update_reps(first, num, int((lens // 64).max()))
    layer.seq_lens.copy_(torch.from_numpy(lens))
    layer.select(H.device_query(cfg, 0), int(lens.max()))
    layer.decode(H.device_q(cfg, 0))
    res = H.fetch(layer)
    for b in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            orow = H.oracle_row(cfg, b, g)
            nb = int(lens[b]) // 64
            H.check_reps(layer, orow, cfg, b, g, nb)
            assert res.num_selected[b, g] == min(k, nb)
            H.check_step(cfg, res, orow, b, g, 0, seq_len=int(lens[b]))
