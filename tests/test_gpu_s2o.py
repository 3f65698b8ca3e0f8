"""S2O prefill on the GPU (nsa_s2o_index + nsa_s2o_attend through the C ABI)
against the CPU oracle: segment orders, stop index per query tile and
outputs, with ragged sequences and segments, both head sizes, group sizes 1
to 8, tau = 0 (dense causal), constructed ties, given orders, and sampled
rows of the 32K-token workload."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import s2o_prefill as S
from tests import s2o_harness as H
from tests.gpu_harness import log

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_all(cfg, pb=None, tag=""):
    log(f"[s2o] {tag or cfg.name}: B={cfg.batch} L={cfg.seq_len} Hq={cfg.num_q_heads} "
        f"Hkv={cfg.num_kv_heads} d={cfg.head_dim} seg={cfg.segment} tau={cfg.tau}")
    r = H.Run(cfg, pb)
    res = r.run()
    stats = [H.check_head(r.pb, res, b, h) for b in range(cfg.batch) for h in range(cfg.num_q_heads)]
    return H.summary(tag or cfg.name, stats), r, res


def test_s2o_tiny():
    tot, _, _ = run_all(W.prefill_config("s2o-tiny"))
    assert tot["n_star_sum"] < tot["n_hist_sum"], "the early stop never fired"


@pytest.mark.parametrize("d,Hq,Hkv", [(64, 4, 2), (128, 8, 1), (128, 2, 2), (64, 8, 8)])
def test_s2o_shapes(d, Hq, Hkv):
    cfg = W.prefill_config("s2o-tiny", cfg_id=42 + Hq + d, head_dim=d, num_q_heads=Hq,
                           num_kv_heads=Hkv, segment=192, seq_len=64 * 11 + 5, len_step=130)
    run_all(cfg, tag=f"d{d}-G{Hq // Hkv}")


def test_s2o_tau_zero_is_dense():
    cfg = W.prefill_config("s2o-tiny", tau=0.0, segment=64, seq_len=64 * 6 + 17)
    tot, _, _ = run_all(cfg, tag="tau0")
    assert tot["n_star_sum"] == tot["n_hist_sum"]


def test_s2o_ties_keep_lower_index():
    """Duplicated keys and queries give equal scores on both sides; equal
    scores must come out lower index first (checked explicitly below: the
    order check alone would accept them either way as a near tie)."""
    cfg = W.prefill_config("s2o-tiny", batch=1, len_step=0)
    pb = W.build_prefill(cfg)
    L = cfg.seq_len
    for b in range(cfg.batch):
        for t in range(300, L, 37):   # copies of token 5's key
            src, dst = pb.table[b, 5 // 64], pb.table[b, t // 64]
            pb.k_pool[dst, :, t % 64] = pb.k_pool[src, :, 5]
        pb.q[b, :, 600:640] = pb.q[b, :, 600:601]   # one query repeated in segment 4
    tot, _, res = run_all(cfg, pb, tag="ties")
    for h in range(cfg.num_q_heads):
        kv = res["kv_perm"][0, h, 6, :768]
        pos = [int(np.flatnonzero(kv == t)[0]) for t in [5] + list(range(300, 768, 37))]
        assert pos == sorted(pos), (h, pos)
        qp = res["q_perm"][0, h, 4]
        at = [int(np.flatnonzero(qp == o)[0]) for o in range(88, 128)]
        assert at == sorted(at), (h, at)


def test_s2o_attend_on_given_orders():
    """nsa_s2o_attend on orders it did not make (seeded random permutations):
    the stop rule and outputs follow the oracle on those orders."""
    cfg = W.prefill_config("s2o-tiny")
    r = H.Run(cfg)
    rng = np.random.default_rng(5)
    qp = np.full(tuple(r.q_perm.shape), -1, dtype=np.int32)
    kp = np.zeros(tuple(r.kv_perm.shape), dtype=np.int32)
    for b in range(cfg.batch):
        L = int(r.pb.seq_lens[b])
        for h in range(cfg.num_q_heads):
            for s in range(r.nseg):
                a = s * cfg.segment
                if a >= L:
                    continue
                n = min(cfg.segment, L - a)
                qp[b, h, s, :n] = rng.permutation(n)
                kp[b, h, s, :a] = rng.permutation(a)
    r.q_perm.copy_(torch.from_numpy(qp))
    r.kv_perm.copy_(torch.from_numpy(kp))
    r.attend()
    torch.cuda.synchronize()
    res = r.fetch()
    stats = []
    for b in range(cfg.batch):
        for h in range(cfg.num_q_heads):
            q, keys, vals = H.head_inputs(r.pb, b, h)
            L = q.shape[0]
            st = {"tiles": 0, "max_err": 0.0}
            for s in range(-(-L // cfg.segment)):
                a = s * cfg.segment
                n = min(cfg.segment, L - a)
                htiles = [kp[b, h, s, i:i + 64].astype(np.int64) for i in range(0, a, 64)]
                for j in range(-(-n // 64)):
                    pos = a + qp[b, h, s, 64 * j:64 * j + 64][: min(64, n - 64 * j)].astype(np.int64)
                    n_gpu = int(res["num_tiles"][b, h, s, j])
                    r_ = H.tile_ratios(q[pos], pos, keys, a, htiles, 1 / np.sqrt(cfg.head_dim),
                                       n_gpu)
                    for t in range(n_gpu - 1):
                        assert np.any(r_[:, t] >= cfg.tau * (1 - H.STOP_MARGIN))
                    if n_gpu < len(htiles):
                        assert np.all(r_[:, n_gpu - 1] < cfg.tau * (1 + H.STOP_MARGIN))
                    kept = np.concatenate(htiles[:n_gpu]) if n_gpu else np.zeros(0, dtype=np.int64)
                    ref = np.stack([S.attend_tokens(q[p], keys, vals,
                                                    np.concatenate([np.arange(a, p + 1), kept]),
                                                    1 / np.sqrt(cfg.head_dim)) for p in pos])
                    err = np.abs(res["out"][b, h, pos] - ref).max()
                    assert err <= H.TOL, (b, h, s, j, err)
                    st["tiles"] += 1
                    st["max_err"] = max(st["max_err"], float(err))
            stats.append(st)
    log(f"[s2o] given orders: {sum(s['tiles'] for s in stats)} query tiles, max-abs "
        f"{max(s['max_err'] for s in stats):.3g}")


def test_s2o_prefill_32k_sampled():
    """The 32K-token workload in the bench's launch: orders of sampled
    segments and stops and outputs of sampled query tiles."""
    cfg = W.prefill_config("s2o-prefill-32k")
    r = H.Run(cfg)
    res = r.run()
    stats = []
    for h, segs in ((0, [1, 17, 31]), (13, [2, 30]), (31, [31])):
        stats.append(H.check_head(r.pb, res, 0, h, segments=segs, tiles=[0, 7, 15]))
    tot = H.summary("s2o-prefill-32k sampled", stats)
    assert tot["n_star_sum"] < tot["n_hist_sum"]
