"""GPU side of the S2O prefill parity tests: upload a seeded prefill, run
nsa_s2o_index and nsa_s2o_attend through the C ABI, and compare with the
CPU oracle.

Acceptance:
  * Q_perm / KV_perm: permutations of the segment's offsets / history
    tokens, in an order the oracle accepts: each adjacent pair (x, y) has
    score(x) > score(y), or equal scores with x < y, or scores within a
    near tie of 2e-5 * max(sum_d |x_d g_d|, sum_d |y_d g_d|) (g the guide
    vector or representative query: the bound of the fp32 dot products'
    rounding, with margin).  The count of entries equal to the oracle's own
    order is reported.
  * stop index n* of each query tile, on the GPU's orders: for every walked
    tile before n*, some query's ratio M/A (fp64) is at least tau*(1 - 1e-3);
    at n* (if the walk stopped) every ratio is below tau*(1 + 1e-3) -- the
    margin covers fp32 masses against fp64.
  * outputs: max-abs 2e-2 against the oracle's attention over exactly the
    tokens the GPU kept (pass 1 plus the first n* history tiles).
"""

from __future__ import annotations

import numpy as np
import torch

import workloads as W
from oracle import s2o_prefill as S
from tests.gpu_harness import log, to_dev

ORDER_TIE = 2e-5
STOP_MARGIN = 1e-3
TOL = 2e-2


def lib():
    import block_sparse_kv_nsa_amd as N
    return N


def round64(n: int) -> int:
    return (n + 63) // 64 * 64


class Run:
    """Device buffers and results of one S2O prefill."""

    def __init__(self, cfg: W.PrefillConfig, pb: W.PrefillBatch | None = None, device="cuda"):
        N = lib()
        self.cfg = cfg
        self.pb = pb if pb is not None else W.build_prefill(cfg)
        B, Hq, Hkv, d, seg = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.segment
        self.max_len = round64(cfg.seq_len)
        self.nseg = -(-self.max_len // seg)
        q = np.zeros((B, Hq, self.max_len, d), dtype=np.uint16)
        q[:, :, :cfg.seq_len] = self.pb.q
        self.q = to_dev(q, "bf16", device)
        self.k_pool = to_dev(self.pb.k_pool, "bf16", device)
        self.v_pool = to_dev(self.pb.v_pool, "bf16", device)
        self.table = torch.from_numpy(self.pb.table).to(device)
        self.seq_lens = torch.from_numpy(self.pb.seq_lens).to(device)
        self.shape = N.Shape.make(B, Hq, Hkv, d, cfg.max_blocks, cfg.num_phys_blocks, N.NSA_BF16)
        self.params = N.PrefillParams(seg, self.max_len, cfg.tau)
        self.ws_bytes = N.nsa_s2o_workspace_bytes(self.shape, self.params)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.q_perm = torch.full((B, Hq, self.nseg, seg), -7, dtype=torch.int32, device=device)
        self.kv_perm = torch.full((B, Hq, self.nseg, self.max_len), -7, dtype=torch.int32,
                                  device=device)
        self.out = torch.zeros((B, Hq, self.max_len, d), dtype=torch.bfloat16, device=device)
        self.num_tiles = torch.full((B, Hq, self.nseg, seg // 64), -7, dtype=torch.int32,
                                    device=device)

    def index(self, stream=None):
        lib().nsa_s2o_index(self.shape, self.params, self.q, self.k_pool, self.table,
                            self.seq_lens, self.q_perm, self.kv_perm, self.ws, self.ws_bytes,
                            stream)

    def attend(self, stream=None, q_perm=None, kv_perm=None):
        lib().nsa_s2o_attend(self.shape, self.params, self.q, self.k_pool, self.v_pool, self.table,
                             self.seq_lens, self.q_perm if q_perm is None else q_perm,
                             self.kv_perm if kv_perm is None else kv_perm, self.out,
                             self.num_tiles, self.ws, self.ws_bytes, stream)

    def run(self):
        self.index()
        self.attend()
        torch.cuda.synchronize()
        return self.fetch()

    def fetch(self):
        return {"q_perm": self.q_perm.cpu().numpy(), "kv_perm": self.kv_perm.cpu().numpy(),
                "num_tiles": self.num_tiles.cpu().numpy(),
                "out": self.out.to(torch.float32).cpu().numpy().astype(np.float64)}


def head_inputs(pb: W.PrefillBatch, b: int, h: int):
    """The head's queries, keys and values (float64), read back from the
    host copies of what was uploaded."""
    cfg = pb.cfg
    L, g = int(pb.seq_lens[b]), h // cfg.group
    t = np.arange(L)
    slots = pb.table[b, t // 64]
    f = lambda a: W.stored_to_f64(a, "bf16")  # noqa: E731
    return f(pb.q[b, h, :L]), f(pb.k_pool[slots, g, t % 64]), f(pb.v_pool[slots, g, t % 64])


def check_order(gpu: np.ndarray, scores: np.ndarray, rows: np.ndarray, vec: np.ndarray, what: str):
    """gpu: the GPU's order; scores: oracle scores of rows against vec."""
    n = scores.size
    assert np.array_equal(np.sort(gpu), np.arange(n)), f"{what}: not a permutation"
    mag = np.abs(rows * vec[None, :]).sum(axis=1)
    x, y = gpu[:-1], gpu[1:]
    sx, sy = scores[x], scores[y]
    ok = (sx > sy) | ((sx == sy) & (x < y)) | (np.abs(sx - sy) <= ORDER_TIE * np.maximum(mag[x], mag[y]))
    bad = np.flatnonzero(~ok)
    assert bad.size == 0, (f"{what}: entries {bad[:5]} out of order: "
                           f"{[(int(x[i]), int(y[i]), sx[i], sy[i]) for i in bad[:3]]}")
    return int((gpu == S.descending_order(scores)).sum())


def tile_ratios(q_rows, positions, keys, start, tiles, scale, upto):
    """M/A of every query (rows) for history tiles 1..upto (fp64)."""
    own = [np.arange(start, int(p) + 1) for p in positions]
    hist = np.concatenate(tiles) if tiles else np.zeros(0, dtype=np.int64)
    out = []
    for i in range(len(q_rows)):
        lg_own = keys[own[i]] @ q_rows[i] * scale
        lg_h = keys[hist] @ q_rows[i] * scale if hist.size else np.zeros(0)
        c = max(lg_own.max(), lg_h.max() if lg_h.size else -np.inf)
        A = np.exp(lg_own - c).sum()
        r = []
        for n in range(upto):
            M = np.exp(lg_h[64 * n:64 * (n + 1)] - c).sum()
            A += M
            r.append(M / A)
        out.append(r)
    return np.array(out).reshape(len(q_rows), upto)


def check_head(pb: W.PrefillBatch, res, b: int, h: int, segments=None, tiles=None) -> dict:
    """Compare one (sequence, query head) with the oracle.  segments / tiles:
    optional subsets (sampling at full size)."""
    cfg = pb.cfg
    q, keys, vals = head_inputs(pb, b, h)
    L, seg, d = q.shape[0], cfg.segment, cfg.head_dim
    scale = 1.0 / np.sqrt(d)
    stats = {"q_equal": 0, "q_total": 0, "kv_equal": 0, "kv_total": 0, "tiles": 0, "max_err": 0.0,
             "n_star_sum": 0, "n_hist_sum": 0}
    segs = range(-(-L // seg)) if segments is None else segments
    for s in segs:
        a = s * seg
        if a >= L:
            continue
        e = min(a + seg, L)
        n = e - a
        gq = res["q_perm"][b, h, s]
        assert np.all(gq[n:] == -1), (b, h, s, "q_perm tail")
        gq = gq[:n].astype(np.int64)
        guide = S.stored_mean(keys[:a], "bf16", d)
        _, qs = S.query_order(q[a:e], keys, a, "bf16")
        stats["q_equal"] += check_order(gq, qs, q[a:e], guide, f"Q_perm b{b} h{h} s{s}")
        stats["q_total"] += n
        gk = res["kv_perm"][b, h, s, :a].astype(np.int64)
        if a:
            rep = S.stored_mean(q[a:e], "bf16", d)
            _, ks = S.history_order(q[a:e], keys, a, "bf16")
            stats["kv_equal"] += check_order(gk, ks, keys[:a], rep, f"KV_perm b{b} h{h} s{s}")
            stats["kv_total"] += a
        htiles = S.history_tiles(gk)
        jt = range(-(-n // 64)) if tiles is None else [j for j in tiles if 64 * j < n]
        for j in jt:
            offs = gq[64 * j:64 * (j + 1)]
            pos = a + offs
            n_gpu = int(res["num_tiles"][b, h, s, j])
            assert 0 <= n_gpu <= len(htiles), (b, h, s, j, n_gpu)
            r = tile_ratios(q[pos], pos, keys, a, htiles, scale, n_gpu)
            for t in range(n_gpu - 1):
                assert np.any(r[:, t] >= cfg.tau * (1 - STOP_MARGIN)), \
                    (f"b{b} h{h} s{s} tile{j}: the oracle stops at history tile {t + 1} "
                     f"but the GPU walked {n_gpu}")
            if n_gpu < len(htiles):
                assert n_gpu >= 1 and np.all(r[:, n_gpu - 1] < cfg.tau * (1 + STOP_MARGIN)), \
                    f"b{b} h{h} s{s} tile{j}: GPU stopped at {n_gpu} without the ratio below tau"
            kept = np.concatenate(htiles[:n_gpu]) if n_gpu else np.zeros(0, dtype=np.int64)
            ref = np.stack([S.attend_tokens(q[p], keys, vals, np.concatenate([np.arange(a, p + 1), kept]),
                                            scale) for p in pos])
            err = np.abs(res["out"][b, h, pos] - ref).max()
            assert err <= TOL, f"b{b} h{h} s{s} tile{j}: max-abs {err:.3g} > {TOL}"
            stats["max_err"] = max(stats["max_err"], float(err))
            stats["tiles"] += 1
            stats["n_star_sum"] += n_gpu
            stats["n_hist_sum"] += len(htiles)
    return stats


def summary(tag: str, stats_list) -> dict:
    tot = {k: sum(s[k] for s in stats_list) for k in stats_list[0] if k != "max_err"}
    tot["max_err"] = max(s["max_err"] for s in stats_list)
    log(f"[{tag}] Q_perm equal {tot['q_equal']}/{tot['q_total']}, KV_perm equal "
        f"{tot['kv_equal']}/{tot['kv_total']}, {tot['tiles']} query tiles, history tiles walked "
        f"{tot['n_star_sum']}/{tot['n_hist_sum']}, max-abs {tot['max_err']:.3g}")
    return tot
