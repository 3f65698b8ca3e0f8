"""Decode steps captured in a HIP graph and replayed: every replay gives the
same selection and the same output bits as the same steps launched one by
one (the library enqueues no memset and leaves its counters and hand-off
slots as it found them, so a captured call needs no clearing in between).

The captured steps are steady-state steps (no block fills in them), so the
eviction state they read does not change from one replay to the next.  Each
replay is separated from the next by unrelated eager work and a
synchronisation, and every replay is checked.
"""

from __future__ import annotations

import pytest
import torch

import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = {
    "fused": dict(ordered=False, tau=0.0, k_e=16, fused=True),
    "split": dict(ordered=False, tau=0.0, k_e=16, fused=False),
    "split-ordered": dict(ordered=True, tau=1e-3, k_e=0, fused=False),
}


def _launch(layer, cfg, lens_t, query_t, q_t, max_len, fused):
    """One step on the current stream from device tensors only (nothing is
    copied from the host, so the calls can be captured)."""
    layer.seq_lens = lens_t
    if fused:
        layer.step(query_t, q_t, max_len)
    else:
        layer.select(query_t, max_len)
        layer.decode(q_t)


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_match_eager_steps(case):
    c = CASES[case]
    cfg = W.Config("graph-" + case, 74, batch=3, context=64 * 150 + 9, num_q_heads=8,
                   num_kv_heads=2, head_dim=128, dtype="bf16", mode="group_softmax",
                   k=32 if c["ordered"] else 24, k_e=c["k_e"], steps=4,
                   ordered=c["ordered"], tau=c["tau"])
    H.log(f"[case] graph capture and replay, {case}")
    batch = W.build_batch(cfg)
    eager, graphed = H.make_layer(cfg, batch), H.make_layer(cfg, batch)
    for lay in (eager, graphed):
        H.prefill(lay, cfg)
        H.run_step(lay, cfg, 0, fused=c["fused"])  # the first step updates the eviction state
    torch.cuda.synchronize()

    dev = eager.device
    steps = range(1, cfg.steps)
    assert all(cfg.seq_len(t) % 64 != 0 for t in steps), "captured steps must not fill a block"
    lens = {t: torch.full((cfg.batch,), cfg.seq_len(t), dtype=torch.int32, device=dev)
            for t in steps}
    queries = {t: H.device_query(cfg, t) for t in steps}
    qs = {t: H.device_q(cfg, t) for t in steps}

    want = {}
    for t in steps:
        _launch(eager, cfg, lens[t], queries[t], qs[t], cfg.seq_len(t), c["fused"])
        torch.cuda.synchronize()
        want[t] = (eager.out.clone(), eager.selected.clone(), eager.num_selected.clone(),
                   eager.num_processed.clone())

    outs = {t: torch.empty_like(graphed.out) for t in steps}
    sels = {t: torch.empty_like(graphed.selected) for t in steps}
    nsel = {t: torch.empty_like(graphed.num_selected) for t in steps}
    nproc = {t: torch.empty_like(graphed.num_processed) for t in steps}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in steps:
            _launch(graphed, cfg, lens[t], queries[t], qs[t], cfg.seq_len(t), c["fused"])
            outs[t].copy_(graphed.out)
            sels[t].copy_(graphed.selected)
            nsel[t].copy_(graphed.num_selected)
            nproc[t].copy_(graphed.num_processed)
    torch.cuda.synchronize()

    x = torch.randn(512, 512, device=dev)
    for rep in range(3):
        for t in steps:
            for buf in (outs[t], sels[t], nsel[t], nproc[t]):
                buf.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t in steps:
            o, s, n, p = want[t]
            assert torch.equal(nsel[t], n), (case, rep, t)
            assert torch.equal(sels[t], s), (case, rep, t)
            if c["ordered"]:
                assert torch.equal(nproc[t], p), (case, rep, t)
            assert torch.equal(outs[t].view(torch.int16), o.view(torch.int16)), (case, rep, t)
        if c["fused"]:
            H.check_step_status(graphed)
        # unrelated eager work between replays
        x = torch.tanh(x @ x * 1e-3)
        torch.cuda.synchronize()
    del graph
