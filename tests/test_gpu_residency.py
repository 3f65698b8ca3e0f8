"""GPU parity of the residency diff (nsa_residency_diff) against the CPU
oracle's set difference: fetch and release lists bit-exact, gamma exact.

Every case prints what it runs before touching the GPU.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import nsa_oracle as O
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_diff(N, shape, ms, prev, prev_num, prev_lens, cur, num):
    dev = "cuda"
    B, Hkv = prev_num.shape
    fetch = torch.full((B, Hkv, ms), 7, dtype=torch.int32, device=dev)
    release = torch.full((B, Hkv, ms + 1), 7, dtype=torch.int32, device=dev)
    nf = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
    nr = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
    gamma = torch.zeros((B, Hkv), dtype=torch.float32, device=dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    N.nsa_residency_diff(shape, ms, t(prev), t(prev_num), t(prev_lens), t(cur), t(num), fetch, nf,
                         release, nr, gamma)
    torch.cuda.synchronize()
    return fetch.cpu().numpy(), nf.cpu().numpy(), release.cpu().numpy(), nr.cpu().numpy(), \
        gamma.cpu().numpy()


def expect_row(res, b, g, sel, prev, tail, ms):
    fetch, nf, release, nr, gamma = res
    wf, wr = O.residency_diff(sel, prev, tail)
    assert nf[b, g] == len(wf) and fetch[b, g, :nf[b, g]].tolist() == wf.tolist(), (b, g)
    assert nr[b, g] == len(wr) and release[b, g, :nr[b, g]].tolist() == wr.tolist(), (b, g)
    assert (fetch[b, g, nf[b, g]:] == -1).all() and (release[b, g, nr[b, g]:] == -1).all()
    S = np.unique(np.asarray(sel, dtype=np.int64))
    want_g = np.float32(len(S) - len(wf)) / np.float32(len(S)) if len(S) else np.float32(1)
    assert gamma[b, g] == want_g, (gamma[b, g], want_g)


@pytest.mark.parametrize("max_blocks,ms", [(50, 16), (2049, 64), (16384, 300)])
def test_random_sets(max_blocks, ms):
    """Random, unsorted, repeated and out-of-range ids; tails present or not."""
    H.log(f"[case] residency diff random sets max_blocks={max_blocks} k={ms}")
    N = H.lib()
    B, Hkv = 3, 4
    shape = N.Shape.make(B, Hkv * 2, Hkv, 64, max_blocks, B * max_blocks, N.NSA_BF16)
    rng = np.random.default_rng(max_blocks)
    prev = rng.integers(-3, max_blocks + 3, (B, Hkv, ms))
    cur = rng.integers(-3, max_blocks + 3, (B, Hkv, ms))
    # overlapping selections, as consecutive steps have
    cur[..., : ms // 2] = prev[..., ms // 4: ms // 4 + ms // 2]
    prev_num = rng.integers(0, ms + 1, (B, Hkv))
    num = rng.integers(0, ms + 1, (B, Hkv))
    num[0, 0] = 0
    prev_lens = np.array([64 * (max_blocks // 2), 64 * (max_blocks // 3) + 5, 17])
    res = run_diff(N, shape, ms, prev, prev_num, prev_lens, cur, num)
    for b in range(B):
        L = int(prev_lens[b])
        tail = L // 64 if L % 64 else None
        if tail is not None and tail >= max_blocks:
            tail = None
        for g in range(Hkv):
            ok = lambda v: [int(x) for x in v if 0 <= x < max_blocks]
            expect_row(res, b, g, ok(cur[b, g, :num[b, g]]), ok(prev[b, g, :prev_num[b, g]]),
                       tail, ms)


@pytest.mark.parametrize("fused", [False, True])
def test_decode_trajectory(fused):
    """Config 1 (160 steps, blocks filling at steps 63 and 127): the diff of
    the library's consecutive selections equals the oracle's, and gamma
    stays at or above k_e / k."""
    cfg = W.config(1, steps=160, batch=2)
    H.log(f"[case] residency diff over {cfg.name} x {cfg.steps} steps fused={fused}")
    N = H.lib()
    batch = W.build_batch(cfg)
    layer = H.make_layer(cfg, batch)
    H.prefill(layer, cfg)
    prev_sel = prev_num = prev_lens = None
    g_min = 1.0
    for t in range(cfg.steps):
        H.run_step(layer, cfg, t, fused=fused)
        L = cfg.seq_len(t)
        if prev_sel is not None:
            res = run_diff(N, layer.shape, cfg.k, prev_sel, prev_num, prev_lens,
                           layer.selected.cpu().numpy(), layer.num_selected.cpu().numpy())
            cur = layer.selected.cpu().numpy()
            num = layer.num_selected.cpu().numpy()
            tail = (L - 1) // 64 if (L - 1) % 64 else None
            for b in range(cfg.batch):
                for g in range(cfg.num_kv_heads):
                    expect_row(res, b, g, cur[b, g, :num[b, g]], prev_sel[b, g, :prev_num[b, g]],
                               tail, cfg.k)
            g_min = min(g_min, float(res[4].min()))
        prev_sel = layer.selected.cpu().numpy()
        prev_num = layer.num_selected.cpu().numpy()
        prev_lens = np.full(cfg.batch, L, dtype=np.int32)
    if fused:
        layer.check_step()
    assert g_min >= cfg.k_e / cfg.k, g_min
