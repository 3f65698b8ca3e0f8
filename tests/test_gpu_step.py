"""GPU parity of the fused decode step (nsa_decode_step) against the CPU oracle,
and against the two-call path (nsa_select_blocks + nsa_sparse_decode).

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


def test_step_config0_tiny_fp32():
    H.run_and_check(W.config(0), fused=True)


def test_step_config1_all_rows():
    _, st = H.run_and_check(W.config(1), fused=True)
    assert st["gamma_min"] >= 0.75


def test_step_config1_fill_steps():
    cfg = W.config(1, steps=160, batch=4)
    _, st = H.run_and_check(cfg, check_every=3, fused=True)
    assert st["gamma_min"] >= 0.75


def test_step_config2_forecast_sampled_rows():
    cfg = W.config(2)
    H.run_and_check(cfg, rows=H.sample_rows(cfg, 12), fused=True)


def test_step_config2_inference_window_sampled_rows():
    cfg = W.config(2).replace(name="sparda-8b-window", mode="forecast_window")
    H.run_and_check(cfg, rows=H.sample_rows(cfg, 12), fused=True)


def test_step_config3_long_context_sampled_rows():
    cfg = W.config(3)
    _, st = H.run_and_check(cfg, rows=H.sample_rows(cfg, 6), check_every=3, fused=True)
    assert st["gamma_min"] >= 0.75


def test_step_config3_fill_steps():
    """Config 3 for 80 steps on the fused step: block 2048 fills at step 63
    (the non-steady eviction update inside the kernel at nb = 2049, with a
    split gang, and the selection over a row longer than 2048 blocks)."""
    cfg = W.config(3, steps=80)
    _, st = H.run_and_check(cfg, rows=H.sample_rows(cfg, 4), check_every=8, fused=True)
    assert st["gamma_min"] >= 0.75


def test_step_status_query_reports_no_expiry():
    """nsa_decode_step_status on a workspace whose steps all completed:
    NSA_OK, and the query leaves the workspace usable."""
    cfg = W.config(0)
    layer, _ = H.run_and_check(cfg, fused=True)
    layer.check_step()
    H.run_step(layer, cfg, 0, fused=True)
    layer.check_step()


SMALL = [
    ("f32", 64, 1, "group_softmax"),
    ("f32", 128, 2, "group_softmax"),
    ("bf16", 64, 8, "group_softmax"),
    ("bf16", 128, 4, "group_softmax"),
    ("bf16", 128, 8, "group_softmax"),
    ("bf16", 128, 4, "forecast"),
    ("f32", 64, 4, "forecast"),
    ("bf16", 64, 1, "forecast"),
    ("bf16", 128, 4, "forecast_window"),
    ("f32", 64, 2, "forecast_window"),
]


@pytest.mark.parametrize("dtype,D,G,mode", SMALL)
def test_step_small_shapes(dtype, D, G, mode):
    cfg = W.Config(f"step-small-{dtype}-{D}-{G}-{mode}", 60 + SMALL.index((dtype, D, G, mode)),
                   batch=3, context=64 * 41 + 37, num_q_heads=2 * G, num_kv_heads=2,
                   head_dim=D, dtype=dtype, mode=mode, k=12, k_e=0 if mode.startswith("forecast") else 8,
                   steps=30)
    H.run_and_check(cfg, fused=True)


def test_step_multi_chunk_rows():
    """Rows of 300 blocks (1200 representatives): several gang members, the
    last with a ragged share."""
    cfg = W.Config("step-chunks", 70, batch=2, context=64 * 300 + 5, num_q_heads=8,
                   num_kv_heads=2, head_dim=128, dtype="bf16", mode="group_softmax", k=40,
                   k_e=24, steps=3)
    H.run_and_check(cfg, fused=True)


@pytest.mark.parametrize("gang", ["1", "3", "5", "64"])
def test_step_gang_sizes(gang, monkeypatch):
    """Any gang size gives the oracle's answer: the smallest allowed (3
    members for 1200 representatives), odd sizes with ragged shares, and 64
    members, where 12 rows exceed the resident gangs and gangs take several
    rows in turn."""
    cfg = W.Config("step-gangs", 73, batch=6, context=64 * 300 + 5, num_q_heads=8,
                   num_kv_heads=2, head_dim=128, dtype="bf16", mode="group_softmax", k=40,
                   k_e=24, steps=2)
    monkeypatch.setenv("NSA_STEP_GANG", gang)
    H.run_and_check(cfg, rows=H.sample_rows(cfg, 5), fused=True)


def test_step_rows_beyond_2048_blocks():
    """Rows of 2600 full blocks: every thread takes several of the row's keys
    in the radix select, and the gang has many members."""
    cfg = W.Config("step-long-rows", 78, batch=1, context=64 * 2600 + 11, num_q_heads=8,
                   num_kv_heads=2, head_dim=128, dtype="bf16", mode="group_softmax", k=40,
                   k_e=24, steps=2)
    H.run_and_check(cfg, fused=True)


def test_step_one_workspace_across_max_seq_len():
    """One workspace, calls whose max_seq_len changes (the per-row key slots
    change stride): every call still gives the oracle's answer."""
    cfg = W.Config("step-maxlen", 79, batch=3, context=64 * 150 + 60, num_q_heads=8,
                   num_kv_heads=2, head_dim=128, dtype="bf16", mode="group_softmax", k=24,
                   k_e=16, steps=6)
    cap = 64 * cfg.max_blocks
    bounds = [cfg.seq_len(0), cap, cfg.seq_len(2), cap, cfg.seq_len(4) + 64 * 3, cfg.seq_len(5)]
    H.run_and_check(cfg, fused=True, max_len=lambda t: min(bounds[t], cap))


def test_step_equal_scores_take_the_lowest_ids():
    """Every key equal, so every block scores the same: the query-aware part is
    the lowest-numbered blocks outside the eviction set (ties to the lower
    id), and the fused call agrees with the two calls."""
    cfg = W.Config("step-ties", 76, batch=2, context=64 * 600 + 5, num_q_heads=8, num_kv_heads=2,
                   head_dim=128, dtype="bf16", mode="group_softmax", k=40, k_e=24, steps=1)
    H.log("[case] fused step, all keys equal")
    batch = W.build_batch(cfg)
    batch.k_pool[...] = batch.k_pool.reshape(-1)[1]
    split, fused = H.make_layer(cfg, batch), H.make_layer(cfg, batch)
    H.prefill(split, cfg)
    H.prefill(fused, cfg)
    H.run_step(split, cfg, 0)
    H.run_step(fused, cfg, 0, fused=True)
    assert H.step_error_word(fused) == 0
    rs, rf = H.fetch(split), H.fetch(fused)
    nb = cfg.seq_len(0) // 64
    assert np.array_equal(rs.evict_set, rf.evict_set)
    for b in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            ev = set(int(x) for x in rf.evict_set[b, g, :cfg.k_e])
            sel = [int(x) for x in rf.selected[b, g, :rf.num_selected[b, g]]]
            want_q = [i for i in range(nb) if i not in ev][:cfg.k - cfg.k_e]
            assert sorted(set(sel) - ev) == want_q, (b, g)
            assert np.array_equal(rs.selected[b, g], rf.selected[b, g]), (b, g)
    assert np.abs(rs.out - rf.out).max() <= 1e-2


@pytest.mark.parametrize("k,k_e", [(8, 4), (8, 8), (8, 0)])
def test_step_ragged_batch_edges(k, k_e):
    cfg = W.Config("ragged", 50, batch=5, context=64 * 24, num_q_heads=8, num_kv_heads=2,
                   head_dim=128, dtype="bf16", mode="group_softmax", k=k, k_e=k_e, steps=1)
    lens = np.array([37, 64, 64 * 5 + 1, 64 * 20, 64 * 3], dtype=np.int32)
    H.log(f"[case] fused, ragged seq_lens {lens.tolist()} k={k} k_e={k_e}")
    batch = W.build_batch(cfg)
    layer = H.make_layer(cfg, batch)
    first = torch.zeros(cfg.batch, dtype=torch.int32, device="cuda")
    num = torch.from_numpy(lens // 64).to("cuda")
    layer.update_reps(first, num, int((lens // 64).max()))
    layer.seq_lens.copy_(torch.from_numpy(lens))
    layer.step(H.device_query(cfg, 0), H.device_q(cfg, 0), int(lens.max()))
    assert H.step_error_word(layer) == 0
    res = H.fetch(layer)
    for b in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            orow = H.oracle_row(cfg, b, g)
            assert res.num_selected[b, g] == min(k, int(lens[b]) // 64)
            H.check_step(cfg, res, orow, b, g, 0, seq_len=int(lens[b]))


def test_step_rows_filled_to_capacity():
    """Sequences whose every block slot is full (no tail block): the table
    row is read up to its last entry and no further."""
    cfg = W.Config("full-rows", 51, batch=3, context=64 * 24 - 1, num_q_heads=8, num_kv_heads=2,
                   head_dim=128, dtype="bf16", mode="group_softmax", k=8, k_e=4, steps=1)
    cap = 64 * cfg.max_blocks
    assert cap == cfg.total_tokens
    lens = np.array([cap, cap - 64, 64 * 7], dtype=np.int32)
    H.log(f"[case] fused, rows filled to capacity seq_lens {lens.tolist()}")
    batch = W.build_batch(cfg)
    layer = H.make_layer(cfg, batch)
    first = torch.zeros(cfg.batch, dtype=torch.int32, device="cuda")
    num = torch.from_numpy(lens // 64).to("cuda")
    layer.update_reps(first, num, int((lens // 64).max()))
    layer.seq_lens.copy_(torch.from_numpy(lens))
    layer.step(H.device_query(cfg, 0), H.device_q(cfg, 0), int(lens.max()))
    assert H.step_error_word(layer) == 0
    res = H.fetch(layer)
    for b in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            orow = H.oracle_row(cfg, b, g)
            H.check_step(cfg, res, orow, b, g, 0, seq_len=int(lens[b]))


def _two_layers(cfg):
    batch = W.build_batch(cfg)
    a, b = H.make_layer(cfg, batch), H.make_layer(cfg, batch)
    H.prefill(a, cfg)
    H.prefill(b, cfg)
    return a, b


def test_step_agrees_with_two_calls_and_clears_its_slots():
    """Same selection and eviction state as select + decode; outputs within
    one bf16 rounding where the sets agree; the hand-off slots back at zero
    after every call (so the next call needs no clearing)."""
    cfg = W.Config("step-vs-split", 71, batch=3, context=64 * 200 + 9, num_q_heads=8,
                   num_kv_heads=2, head_dim=128, dtype="bf16", mode="group_softmax", k=24,
                   k_e=16, steps=70)
    H.log("[case] fused step vs two calls, 70 steps")
    split, fused = _two_layers(cfg)
    same_rows = 0
    for t in range(cfg.steps):
        H.run_step(split, cfg, t)
        H.run_step(fused, cfg, t, fused=True)
        assert H.step_error_word(fused) == 0
        slots = H.step_slot_words(fused, cfg)
        assert int(torch.count_nonzero(slots)) == 0, "hand-off slots not cleared"
        rs, rf = H.fetch(split), H.fetch(fused)
        assert np.array_equal(rs.evict_set, rf.evict_set)
        for b in range(cfg.batch):
            for g in range(cfg.num_kv_heads):
                if np.array_equal(rs.selected[b, g], rf.selected[b, g]):
                    same_rows += 1
                    G = cfg.group
                    d = np.abs(rs.out[b, g * G:(g + 1) * G] - rf.out[b, g * G:(g + 1) * G]).max()
                    assert d <= 1e-2, (t, b, g, d)
    assert same_rows >= 0.9 * cfg.steps * cfg.rows


def test_step_rejects_ordered_mode():
    cfg = W.Config("step-ordered", 72, batch=1, context=64 * 10, num_q_heads=4, num_kv_heads=1,
                   head_dim=128, dtype="bf16", mode="group_softmax", k=8, k_e=0, steps=1,
                   ordered=True, tau=1e-3)
    H.log("[case] fused step in ordered mode must be refused")
    layer = H.make_layer(cfg, W.build_batch(cfg))
    with pytest.raises(Exception):
        layer.step(H.device_query(cfg, 0), H.device_q(cfg, 0), cfg.seq_len(0))
