"""Pins for the S2O prefill oracle: checks against things other than the
oracle itself.

Each ``check_*`` takes the oracle module (or a copy with one function swapped
for a planted mistake) and raises AssertionError when it disagrees with a
library routine (torch's attention and softmax in float64), brute force
(exact rational means and orders by counting), a closed form (tau = 0 is
dense causal attention; a tau above 1 keeps one history tile) or an
invariant (the stop index does not grow with tau).
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

from tests.oracle_pins import nearest_even_by_search

SCALE = 0.35


def dyadic(rng, shape, lo=-2.0, hi=2.0, step=0.25):
    """Values on a grid of quarters: exact in bf16 and in float64 sums."""
    n = int(round((hi - lo) / step))
    return lo + step * rng.integers(0, n + 1, size=shape).astype(np.float64)


def small_head(seed, L=150, d=8):
    rng = np.random.default_rng(seed)
    return dyadic(rng, (L, d)), dyadic(rng, (L, d)), dyadic(rng, (L, d))


def sdpa(q, k, v, mask=None, causal=False):
    """torch's scaled_dot_product_attention on the CPU in float64."""
    tq = torch.tensor(q, dtype=torch.float64)[None, None]
    tk = torch.tensor(k, dtype=torch.float64)[None, None]
    tv = torch.tensor(v, dtype=torch.float64)[None, None]
    m = None if mask is None else torch.tensor(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal,
                                                         scale=SCALE)
    return o[0, 0].numpy()


def exact_bf16_mean(rows):
    """Mean of rows as exact rationals, rounded to 8 significant bits by search."""
    rows = np.asarray(rows)
    n, d = rows.shape
    if n == 0:
        return [Fraction(0)] * d
    return [nearest_even_by_search(sum((Fraction(float(x)) for x in rows[:, c]), Fraction(0)) / n, 8)
            for c in range(d)]


def order_by_counting(scores):
    """Position i goes to rank #{j : s_j > s_i or (s_j == s_i and j < i)}."""
    n = len(scores)
    out = [None] * n
    for i in range(n):
        r = sum(1 for j in range(n) if scores[j] > scores[i] or (scores[j] == scores[i] and j < i))
        out[r] = i
    return np.array(out, dtype=np.int64)


def brute_orders(q, keys, seg):
    """Q_perm and KV_perm of every segment from exact rational arithmetic."""
    L = q.shape[0]
    qp, kp = [], []
    for a in range(0, L, seg):
        b = min(a + seg, L)
        guide = exact_bf16_mean(keys[:a])
        rep = exact_bf16_mean(q[a:b])
        qs = [sum(Fraction(float(x)) * g for x, g in zip(q[i], guide)) for i in range(a, b)]
        ks = [sum(Fraction(float(x)) * r for x, r in zip(keys[t], rep)) for t in range(a)]
        qp.append(order_by_counting(qs))
        kp.append(order_by_counting(ks))
    return qp, kp


# ----------------------------------------------------------------------------
def check_s2o_orders_brute_force(S):
    """Q_perm and KV_perm equal orders by counting on exact rational scores
    (rational means rounded by search), with ragged segments."""
    for seed, L, seg in ((1, 45, 16), (2, 70, 32)):
        q, k, _ = small_head(seed, L=L, d=5)
        res = S.prefill_head(q, k, k, seg, 0.0, SCALE, "bf16")
        qp, kp = brute_orders(q, k, seg)
        for s in range(len(qp)):
            assert np.array_equal(res["q_perm"][s], qp[s]), ("Q_perm", seed, s)
            assert np.array_equal(res["kv_perm"][s], kp[s]), ("KV_perm", seed, s)


def check_s2o_ties_and_identity(S):
    """Equal scores keep ascending order: segment 0 (no history) keeps its
    queries in order, identical queries keep theirs, duplicated keys are
    listed lower position first."""
    rng = np.random.default_rng(7)
    d, seg = 4, 16
    k = dyadic(rng, (48, d))
    k[20] = k[3]
    k[35] = k[3]
    q = dyadic(rng, (48, d))
    q[32:48] = q[40]            # segment 2: every query the same
    res = S.prefill_head(q, k, k, seg, 0.0, SCALE, "bf16")
    assert np.array_equal(res["q_perm"][0], np.arange(16))
    assert np.array_equal(res["q_perm"][2], np.arange(16))
    for s, order in enumerate(res["kv_perm"]):
        pos = {int(t): i for i, t in enumerate(order)}
        if 35 in pos:
            assert pos[3] < pos[20] < pos[35]
        elif 20 in pos:
            assert pos[3] < pos[20]


def check_s2o_tau_zero_is_dense_causal(S):
    """tau = 0 never stops: every query gets dense causal attention (torch,
    float64), whatever the orders, and every history tile is walked."""
    for seed, L, seg in ((3, 150, 64), (4, 200, 128)):
        q, k, v = small_head(seed, L=L)
        res = S.prefill_head(q, k, v, seg, 0.0, SCALE, "bf16")
        ref = sdpa(q, k, v, causal=True)
        assert np.abs(res["out"] - ref).max() < 1e-12
        for s, stars in enumerate(res["n_star"]):
            assert all(n == -(-s * seg // 64) for n in stars), (s, stars)


def check_s2o_large_tau_keeps_one_tile(S):
    """tau above 1 stops after the first history tile (a tile's mass never
    exceeds the accumulated mass): query p attends tokens [start, p] plus the
    first 64 tokens of the counted order, checked with torch's masked
    attention."""
    q, k, v = small_head(5, L=150, d=6)
    seg = 64
    res = S.prefill_head(q, k, v, seg, 1.5, SCALE, "bf16")
    _, kp = brute_orders(q, k, seg)
    L = q.shape[0]
    mask = np.zeros((L, L), dtype=bool)
    for a in range(0, L, seg):
        first = kp[a // seg][:64]
        for p in range(a, min(a + seg, L)):
            mask[p, a:p + 1] = True
            mask[p, first] = True
    ref = sdpa(q, k, v, mask=mask)
    assert np.abs(res["out"] - ref).max() < 1e-12
    for s, stars in enumerate(res["n_star"]):
        assert all(n == (1 if s else 0) for n in stars), (s, stars)


def tile_ratios(q, k, S, res, seg, s, j):
    """For query tile j of segment s: per history tile n, each query's
    softmax weight of tile n among the tokens it has seen through tile n
    (torch softmax in float64)."""
    a = s * seg
    offs = res["q_perm"][s][j * 64:(j + 1) * 64]
    kv = res["kv_perm"][s]
    tiles = [kv[i:i + 64] for i in range(0, len(kv), 64)]
    out = []
    for n in range(len(tiles)):
        seen = np.concatenate(tiles[:n + 1])
        rows = []
        for o in offs:
            p = a + o
            toks = np.concatenate([np.arange(a, p + 1), seen])
            lg = torch.tensor(k[toks] @ q[p] * SCALE, dtype=torch.float64)
            w = torch.softmax(lg, dim=0).numpy()
            rows.append(w[-len(tiles[n]):].sum())
        out.append(np.array(rows))
    return out


def check_s2o_stop_rule_by_softmax(S):
    """The walk stops at the first history tile whose softmax weight among
    the tokens seen so far is below tau for every query of the query tile
    (weights from torch's softmax, not from the oracle's masses)."""
    for seed, tau in ((11, 0.08), (12, 0.03)):
        q, k, v = small_head(seed, L=320, d=6)
        q[:, 0] = 3.0
        k[::7, 0] = 5.0
        seg = 64
        res = S.prefill_head(q, k, v, seg, tau, SCALE, "bf16")
        fired = 0
        for s in range(1, len(res["n_star"])):
            for j, n_star in enumerate(res["n_star"][s]):
                r = tile_ratios(q, k, S, res, seg, s, j)
                first = next((n + 1 for n, x in enumerate(r) if np.all(x < tau)), len(r))
                assert n_star == first, (seed, s, j, n_star, first)
                fired += first < len(r)
        assert fired > 0


def check_s2o_stop_monotone_in_tau(S):
    """A larger tau never walks more history tiles."""
    q, k, v = small_head(13, L=256, d=6)
    q[:, 1] = 3.0
    k[::5, 1] = 4.0
    prev = None
    for tau in (0.0, 0.005, 0.02, 0.05, 0.2, 1.5):
        res = S.prefill_head(q, k, v, 64, tau, SCALE, "bf16")
        stars = [n for ss in res["n_star"] for n in ss]
        if prev is not None:
            assert all(a <= b for a, b in zip(stars, prev)), (tau, stars, prev)
        prev = stars


def check_s2o_output_is_attention_over_kept_tokens(S):
    """Every output row equals torch's attention over exactly the tokens the
    walk kept: [start, p] plus the first n_star history tiles."""
    q, k, v = small_head(17, L=300, d=6)
    q[:, 2] = 3.0
    k[::6, 2] = 5.0
    seg = 64
    res = S.prefill_head(q, k, v, seg, 0.05, SCALE, "bf16")
    L = q.shape[0]
    mask = np.zeros((L, L), dtype=bool)
    for s, a in enumerate(range(0, L, seg)):
        kv = res["kv_perm"][s]
        for j, n_star in enumerate(res["n_star"][s]):
            kept = kv[:64 * n_star]
            for o in res["q_perm"][s][j * 64:(j + 1) * 64]:
                p = a + o
                mask[p, a:p + 1] = True
                mask[p, kept] = True
    ref = sdpa(q, k, v, mask=mask)
    assert np.abs(res["out"] - ref).max() < 1e-12


def check_s2o_stored_mean_rounding(S):
    """The stored mean equals the exact rational mean rounded to 8
    significant bits by search, on awkward counts (3, 7, 100 rows)."""
    rng = np.random.default_rng(19)
    for n in (3, 7, 100):
        rows = dyadic(rng, (n, 6), step=0.125) + rng.integers(-3, 4, size=(n, 6)) * 2.0 ** -9
        got = S.stored_mean(rows, "bf16", 6)
        ref = [float(x) for x in exact_bf16_mean(rows)]
        assert np.array_equal(got, np.array(ref)), (n, got, ref)
    assert np.array_equal(S.stored_mean(np.zeros((0, 6)), "bf16", 6), np.zeros(6))


ALL_CHECKS = [
    check_s2o_orders_brute_force,
    check_s2o_ties_and_identity,
    check_s2o_tau_zero_is_dense_causal,
    check_s2o_large_tau_keeps_one_tile,
    check_s2o_stop_rule_by_softmax,
    check_s2o_stop_monotone_in_tau,
    check_s2o_output_is_attention_over_kept_tokens,
    check_s2o_stored_mean_rounding,
]
