"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``check_*`` takes the oracle module (or a copy with one function swapped
for a planted mistake) and raises AssertionError when the oracle disagrees
with brute force, a closed form, a library routine or a hand-worked fixture.
``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutants.py``
plants mistakes in copies of the oracle and requires some check to fail.
"""

from __future__ import annotations

import itertools
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# independent helpers (search-based rounding, loop-based arithmetic)
# ----------------------------------------------------------------------------
def nearest_even_by_search(q: Fraction, bits: int) -> Fraction:
    """Round by listing the representable neighbours and comparing distances."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - bits + 1)
    lo_n = math.floor(a / ulp)
    best = None
    for n in (lo_n, lo_n + 1):
        c = n * ulp
        dist = abs(a - c)
        key = (dist, n % 2)          # nearer first, then even significand
        if best is None or key < best[0]:
            best = (key, c)
    return best[1] if q > 0 else -best[1]


def fsum_exact(vals) -> Fraction:
    return sum((Fraction(float(v)) for v in vals), Fraction(0))


def load_golden_rounding():
    rows = []
    with open(os.path.join(GOLDEN, "bf16_rounding.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            x, y = line.split()[:2]
            rows.append((float.fromhex(x), float.fromhex(y)))
    return rows


def load_golden_selection():
    S = np.array([0.5, 0.9, 0.9, 0.1, 0.7, 0.9, 0.2, 0.7])
    E = np.array([3, 1, 2, 2, 0, 5, 1, 2], dtype=np.float64)
    cases = []
    with open(os.path.join(GOLDEN, "selection_cases.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, k, k_e, ordered, ev, sel = line.split()
            parse = (lambda s: [] if s == "-" else [int(v) for v in s.split(",")])
            cases.append(dict(name=name, k=int(k), k_e=int(k_e), ordered=bool(int(ordered)),
                              evict=parse(ev), selected=parse(sel)))
    return S, E, cases


# ----------------------------------------------------------------------------
# rounding
# ----------------------------------------------------------------------------
def check_round(O):
    for x, y in load_golden_rounding():
        got = float(O.round_bf16(np.array([x]))[0])
        assert got == y, (x.hex(), got.hex(), y.hex())
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.standard_normal(300) * 10.0 ** rng.integers(-6, 6, 300),
                         rng.standard_normal(100)])
    rb = O.round_bf16(xs)
    rf = O.round_f32(xs)
    for x, a, b in zip(xs, rb, rf):
        assert a == float(nearest_even_by_search(Fraction(float(x)), 8)), x
        assert b == float(nearest_even_by_search(Fraction(float(x)), 24)), x
    # library routine: float32 -> bfloat16 in torch rounds to nearest even
    import torch
    x32 = rng.standard_normal(2000).astype(np.float32)
    lib = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x32.astype(np.float64)), lib)


def check_rne_fraction(O):
    rng = np.random.default_rng(12)
    for _ in range(300):
        q = Fraction(int(rng.integers(-10**9, 10**9)), int(rng.integers(1, 10**6)))
        for bits in (8, 24):
            assert O.rne_fraction(q, bits) == nearest_even_by_search(q, bits)
    # exact ties
    assert O.rne_fraction(Fraction(257, 256), 8) == 1
    assert O.rne_fraction(Fraction(259, 256), 8) == Fraction(260, 256)


def check_rounded_means(O):
    rng = np.random.default_rng(13)
    cases = [rng.standard_normal((40, 16))]
    wide = rng.standard_normal((20, 16))
    wide[:, 3] *= 1e-12            # exponent spans beyond float64's 53 bits
    wide[:, 7] *= 1e12
    cases.append(wide)
    for x in cases:
        for storage, bits in (("bf16", 8), ("f32", 24)):
            xs = x.astype(np.float32).astype(np.float64)
            got = O.rounded_means(xs, storage)
            for i in range(xs.shape[0]):
                want = nearest_even_by_search(fsum_exact(xs[i]) / 16, bits)
                assert got[i] == float(want), (storage, i)


# ----------------------------------------------------------------------------
# step 1: representatives and eviction scores
# ----------------------------------------------------------------------------
def check_reps_layout(O):
    """Integer keys: every sub-block mean is a multiple of 1/16 below 16 in
    magnitude, exact in bf16, so the representative is the plain mean of the
    right 16 tokens."""
    rng = np.random.default_rng(14)
    nb, d = 5, 6
    keys = rng.integers(-8, 9, size=(nb * 64 + 17, d)).astype(np.float64)
    reps = O.block_reps(keys, nb, "bf16")
    assert reps.shape == (nb, 4, d)
    for b in range(nb):
        for j in range(4):
            for c in range(d):
                toks = [keys[64 * b + 16 * j + i, c] for i in range(16)]
                assert reps[b, j, c] == sum(toks) / 16.0
    # linearity: the mean of per-token scores equals the score of the mean key
    q = rng.standard_normal(d)
    for b in range(nb):
        for j in range(4):
            tok = keys[64 * b + 16 * j: 64 * b + 16 * j + 16]
            assert abs(np.mean(tok @ q) - reps[b, j] @ q) < 1e-12


def check_eviction_scores(O):
    rng = np.random.default_rng(15)
    nb = 6
    logits = rng.standard_normal(nb * 64 + 5).astype(np.float32).astype(np.float64)
    E = O.eviction_block_scores(logits, nb)
    for b in range(nb):
        means = [fsum_exact(logits[64 * b + 16 * j: 64 * b + 16 * j + 16]) / 16 for j in range(4)]
        assert E[b] == float(nearest_even_by_search(max(means), 24))


# ----------------------------------------------------------------------------
# step 2: scores
# ----------------------------------------------------------------------------
def brute_group_softmax_from_tokens(q, keys, nb, scale):
    """Token-level route: per-token logits, sub-block average of the logits,
    per-head softmax over all sub-blocks, head sum, block maximum."""
    G = len(q)
    nsub = 4 * nb
    sub_logit = [[0.0] * nsub for _ in range(G)]
    for h in range(G):
        for j in range(nsub):
            acc = 0.0
            for i in range(16):
                t = 16 * j + i
                acc += sum(q[h][c] * keys[t][c] for c in range(len(q[h]))) * scale
            sub_logit[h][j] = acc / 16.0
    group = [0.0] * nsub
    for h in range(G):
        mx = max(sub_logit[h])
        z = sum(math.exp(v - mx) for v in sub_logit[h])
        for j in range(nsub):
            group[j] += math.exp(sub_logit[h][j] - mx) / z
    return [max(group[4 * b: 4 * b + 4]) for b in range(nb)]


def check_scores_bruteforce(O):
    rng = np.random.default_rng(16)
    for G, nb, d in ((1, 3, 4), (2, 5, 3), (3, 8, 8)):
        keys = rng.standard_normal((nb * 64, d))
        q = rng.standard_normal((G, d))
        exact = keys.reshape(nb, 4, 16, d).mean(axis=2)      # unrounded means
        S = O.block_scores_group_softmax(q, exact, 0.37)
        want = brute_group_softmax_from_tokens(q.tolist(), keys.tolist(), nb, 0.37)
        assert np.allclose(S, want, rtol=1e-12, atol=0), (G, nb, d)


def check_scores_closed_forms(O):
    rng = np.random.default_rng(17)
    # all representatives equal: every sub-block gets probability 1/(4nb) per
    # head, so every block scores G/(4nb)
    for G, nb in ((1, 7), (4, 16), (8, 3)):
        r = np.tile(rng.standard_normal(5), (nb, 4, 1))
        S = O.block_scores_group_softmax(rng.standard_normal((G, 5)), r, 0.5)
        assert np.allclose(S, G / (4 * nb), rtol=1e-13)
    # one head: softmax is monotone, so blocks rank as their best raw logit
    nb, d = 40, 8
    r = rng.standard_normal((nb, 4, d))
    q = rng.standard_normal((1, d))
    S = O.block_scores_group_softmax(q, r, 0.3)
    raw = (r @ q[0]).max(axis=1)
    assert list(np.argsort(-S, kind="stable")) == list(np.argsort(-raw, kind="stable"))
    # two sub-blocks only can win: logits a and 0 elsewhere, one head
    nb = 3
    r = np.zeros((nb, 4, 1))
    r[1, 2, 0] = 2.0
    S = O.block_scores_group_softmax(np.array([[1.0]]), r, 1.0)
    z = math.exp(2.0) + (4 * nb - 1)
    assert math.isclose(S[1], math.exp(2.0) / z, rel_tol=1e-14)
    assert math.isclose(S[0], 1.0 / z, rel_tol=1e-14)
    assert math.isclose(S[2], 1.0 / z, rel_tol=1e-14)


def check_forecast(O):
    rng = np.random.default_rng(18)
    d, nb = 6, 4
    f = rng.standard_normal(d)
    r = np.zeros((nb, 4, d))
    for b in range(nb):
        for j in range(4):
            r[b, j, (b + j) % d] = 1.0          # basis vectors pick f components
    S = O.block_scores_forecast(f, r)
    for b in range(nb):
        assert S[b] == max(f[(b + j) % d] for j in range(4))
    r = rng.standard_normal((nb, 4, d))
    S = O.block_scores_forecast(f, r)
    for b in range(nb):
        want = max(sum(f[c] * r[b, j, c] for c in range(d)) for j in range(4))
        assert math.isclose(S[b], want, rel_tol=1e-12)


def check_forecast_window(O):
    """The (32, 16) inference window: brute force over the 32-token windows of
    every block from the tokens themselves (unrounded sub-block means), the
    reduction to the raw forecast mode when a block's sub-blocks agree, and a
    window across a block boundary that must not count."""
    rng = np.random.default_rng(19)
    d, nb = 5, 6
    f = rng.standard_normal(d)
    keys = rng.standard_normal((nb * 64, d))
    reps = np.zeros((nb, 4, d))
    for b in range(nb):
        for j in range(4):
            reps[b, j] = sum(keys[64 * b + 16 * j + i] for i in range(16)) / 16.0
    S = O.block_scores_forecast_window(f, reps)
    for b in range(nb):
        best = -math.inf
        for start in (0, 16, 32):
            mean = sum(keys[64 * b + start + i] for i in range(32)) / 32.0
            best = max(best, sum(f[c] * mean[c] for c in range(d)))
        assert math.isclose(S[b], best, rel_tol=1e-12, abs_tol=1e-12), (b, S[b], best)
    same = np.repeat(rng.standard_normal((nb, 1, d)), 4, axis=1)
    assert np.allclose(O.block_scores_forecast_window(f, same), O.block_scores_forecast(f, same),
                       rtol=1e-14, atol=0)
    r = np.zeros((2, 4, 1))
    r[0, 3, 0] = r[1, 0, 0] = 1.0          # only the window across the boundary is 1
    S = O.block_scores_forecast_window(np.array([1.0]), r)
    assert S.tolist() == [0.5, 0.5]


# ----------------------------------------------------------------------------
# step 3: selection
# ----------------------------------------------------------------------------
def exchange_optimal(chosen, cand, score):
    """Every chosen id beats every unchosen one (higher score, or equal score
    and lower id)."""
    out = [c for c in cand if c not in chosen]
    return all(score[a] > score[b] or (score[a] == score[b] and a < b)
               for a in chosen for b in out)


def check_topk_exchange(O):
    rng = np.random.default_rng(19)
    for trial in range(40):
        n = int(rng.integers(1, 9))
        cand = sorted(rng.choice(20, n, replace=False).tolist())
        score = {c: float(rng.integers(0, 4)) for c in cand}   # many exact ties
        for m in range(0, n + 1):
            winners = [set(X) for X in itertools.combinations(cand, m)
                       if exchange_optimal(set(X), cand, score)]
            assert len(winners) == 1
            got = O.top_k(np.array(cand), np.array([score[c] for c in cand]), m)
            assert set(got.tolist()) == winners[0]
            # best first: descending score, ties lower id first
            keys = [(-score[c], c) for c in got.tolist()]
            assert keys == sorted(keys)


def check_selection_golden(O):
    S, E, cases = load_golden_selection()
    nb = len(S)
    for c in cases:
        if c["ordered"]:
            got = O.select_ordered(S, nb, c["k"])
            assert got.tolist() == c["selected"], c["name"]
            continue
        ev = O.eviction_update(np.zeros(0, dtype=np.int64), 0, nb, E, c["k_e"])
        assert ev.tolist() == c["evict"], c["name"]
        got = O.select_blocks(S, ev, nb, c["k"])
        assert got.tolist() == c["selected"], c["name"]


def check_select_bruteforce(O):
    """Enumerate all subsets: eviction set = exchange-optimal k_e subset by E;
    the rest = exchange-optimal subset by S outside it."""
    rng = np.random.default_rng(20)
    for trial in range(30):
        nb = int(rng.integers(1, 9))
        k = int(rng.integers(1, 7))
        k_e = int(rng.integers(0, k + 1))
        S = rng.integers(0, 5, nb).astype(float)
        E = rng.integers(0, 5, nb).astype(float)
        ids = list(range(nb))
        m_e = min(k_e, nb)
        ev = [set(X) for X in itertools.combinations(ids, m_e)
              if exchange_optimal(set(X), ids, {i: E[i] for i in ids})]
        assert len(ev) == 1
        rest = [i for i in ids if i not in ev[0]]
        m_q = min(k - m_e, len(rest))
        qa = [set(X) for X in itertools.combinations(rest, m_q)
              if exchange_optimal(set(X), rest, {i: S[i] for i in rest})]
        want = sorted(ev[0] | qa[0])
        got_ev = O.eviction_update(np.zeros(0, dtype=np.int64), 0, nb, E, k_e)
        got = O.select_blocks(S, got_ev, nb, k)
        assert sorted(got_ev.tolist()) == sorted(ev[0])
        assert got.tolist() == want
        assert len(got) == min(k, nb)


def check_eviction_incremental(O):
    """With fixed E the incremental set equals the global top-k_e of all full
    blocks at every step (closed form), and no dropped block comes back."""
    rng = np.random.default_rng(21)
    for trial in range(20):
        nb_final = int(rng.integers(2, 40))
        k_e = int(rng.integers(1, 12))
        E = rng.integers(0, 6, nb_final).astype(float)
        cur, seen, dropped = np.zeros(0, dtype=np.int64), 0, set()
        nb = int(rng.integers(0, 4))
        while nb <= nb_final:
            new = O.eviction_update(cur, seen, nb, E, k_e)
            ids = list(range(nb))
            glob = sorted(sorted(ids, key=lambda i: (-E[i], i))[:k_e])
            assert new.tolist() == glob
            assert len(new) == min(k_e, nb)
            newly = set(range(seen, nb))
            assert set(new.tolist()) - newly <= set(cur.tolist())
            assert not (set(new.tolist()) & dropped)
            dropped |= set(cur.tolist()) - set(new.tolist())
            cur, seen = new, nb
            nb += int(rng.integers(1, 4))


# ----------------------------------------------------------------------------
# step 4: attention, early stop, locality
# ----------------------------------------------------------------------------
def check_dense_reduction(O):
    """Selecting every block is dense attention: torch's float64 SDPA on CPU."""
    import torch
    rng = np.random.default_rng(22)
    for L, G, d in ((64 * 5 + 9, 4, 16), (64 * 3, 2, 8), (64 * 7 + 63, 1, 32), (17, 3, 4)):
        keys = rng.standard_normal((L + 30, d))
        vals = rng.standard_normal((L + 30, d))
        q = rng.standard_normal((G, d))
        nb = L // 64
        out = O.sparse_attention(q, keys, vals, list(range(nb)), L, 1 / math.sqrt(d))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None, :],
            torch.from_numpy(keys[:L])[None, None].expand(1, G, L, d),
            torch.from_numpy(vals[:L])[None, None].expand(1, G, L, d))[0, :, 0, :].numpy()
        assert np.allclose(out, ref, rtol=0, atol=1e-12), (L, G, d)
        assert np.allclose(O.dense_attention(q, keys, vals, L, 1 / math.sqrt(d)), ref,
                           rtol=0, atol=1e-12)


def check_attend_loops(O):
    """Tiny case against explicit loops over the exact token set."""
    rng = np.random.default_rng(23)
    L, G, d = 64 * 4 + 3, 2, 3
    keys = rng.standard_normal((L, d))
    vals = rng.standard_normal((L, d))
    q = rng.standard_normal((G, d))
    blocks = [2, 0]
    toks = list(range(128, 192)) + list(range(0, 64)) + list(range(256, 259))
    assert sorted(O.token_set(blocks, L).tolist()) == sorted(toks)
    out = O.sparse_attention(q, keys, vals, blocks, L, 0.7)
    for h in range(G):
        lg = [0.7 * sum(q[h][c] * keys[t][c] for c in range(d)) for t in toks]
        mx = max(lg)
        w = [math.exp(v - mx) for v in lg]
        z = sum(w)
        for c in range(d):
            want = sum(w[i] * vals[t][c] for i, t in enumerate(toks)) / z
            assert math.isclose(out[h][c], want, rel_tol=1e-12, abs_tol=1e-14)


def brute_stop_index(q, keys, order, L, tau, scale):
    """From scratch for every prefix: masses in an unshifted frame."""
    nb = L // 64
    tail = list(range(64 * nb, L))

    def mass(h, toks):
        return sum(math.exp(scale * float(np.dot(q[h], keys[t]))) for t in toks)

    for n in range(1, len(order) + 1):
        stop = True
        for h in range(len(q)):
            acc = mass(h, tail) + sum(mass(h, range(64 * b, 64 * b + 64)) for b in order[:n])
            m = mass(h, range(64 * order[n - 1], 64 * order[n - 1] + 64))
            if not m < tau * acc:
                stop = False
        if stop:
            return n
    return len(order)


def check_attention_bias(O):
    """The ED-DMA bias variant: a bias of log(m_t) weighs token t as m_t
    copies of it (brute force by duplication), a constant bias changes
    nothing, and a block whose tokens carry a vanishing weight stops the walk
    right after it."""
    rng = np.random.default_rng(23)
    G, d, L = 2, 5, 64 * 3 + 11
    q = rng.standard_normal((G, d))
    keys = rng.standard_normal((L, d))
    values = rng.standard_normal((L, d))
    mult = rng.integers(1, 4, size=L)
    blocks = [2, 0]
    got = O.sparse_attention(q, keys, values, blocks, L, 0.4, bias=np.log(mult))
    toks = [t for b in blocks for t in range(64 * b, 64 * b + 64)] + list(range(192, L))
    rep = [t for t in toks for _ in range(mult[t])]
    want = O.attend(q, keys[rep], values[rep], 0.4)
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    plain = O.sparse_attention(q, keys, values, blocks, L, 0.4)
    shifted = O.sparse_attention(q, keys, values, blocks, L, 0.4, bias=np.full(L, 3.7))
    assert np.allclose(plain, shifted, rtol=0, atol=1e-12)
    n0, out0 = O.early_stop_attention(q, keys, values, [1, 2, 0], L, 1e-9, 0.4)
    assert n0 == 3
    n1, out1 = O.early_stop_attention(q, keys, values, [1, 2, 0], L, 1e-9, 0.4,
                                      bias=np.full(L, -2.5))
    assert n1 == 3 and np.allclose(out0, out1, rtol=0, atol=1e-12)
    e = np.zeros(L)
    e[128:192] = -60.0                      # block 2: weight e^-60 per token
    n2, out2 = O.early_stop_attention(q, keys, values, [1, 2, 0], L, 1e-9, 0.4, bias=e)
    assert n2 == 2
    assert np.allclose(out2, O.sparse_attention(q, keys, values, [1, 2], L, 0.4, bias=e),
                       rtol=0, atol=1e-12)


def check_early_stop(O):
    rng = np.random.default_rng(24)
    d, G = 8, 2
    L = 64 * 12 + 5
    keys = rng.standard_normal((L, d))
    vals = rng.standard_normal((L, d))
    q = rng.standard_normal((G, d))
    order = list(rng.permutation(12))
    sc = 1 / math.sqrt(d)
    # tau = 0 never stops: all listed blocks, i.e. dense when all are listed
    n, out = O.early_stop_attention(q, keys, vals, order, L, 0.0, sc)
    assert n == 12
    assert np.allclose(out, O.dense_attention(q, keys, vals, L, sc), atol=1e-12)
    # huge tau stops at the first block, which is kept
    n, out = O.early_stop_attention(q, keys, vals, order, L, 1e9, sc)
    assert n == 1
    assert np.allclose(out, O.sparse_attention(q, keys, vals, order[:1], L, sc), atol=1e-12)
    # brute-force prefix scan at several thresholds
    for tau in (1e-3, 0.02, 0.05, 0.08, 0.12, 0.3):
        n, _ = O.early_stop_attention(q, keys, vals, order, L, tau, sc)
        assert n == brute_stop_index(q, keys, order, L, tau, sc), tau
    # hand-worked: one head, scalar keys.  Tail = 1 token with logit 0 (mass 1);
    # pi_1 = block 0 with logits 0 (mass 64, accumulated 65: 64 < 0.065 fails);
    # pi_2 = block 1 with logits -50 (mass 64e-50 < 1e-3*(65+64e-50)): stop,
    # n* = 2.  Values: tail 1, blocks 0 -> out = 1/(65 + 64e^-50).
    keys1 = np.zeros((129, 1))
    keys1[64:128] = -50.0
    vals1 = np.zeros((129, 1))
    vals1[128] = 1.0
    n, out = O.early_stop_attention(np.array([[1.0]]), keys1, vals1, [0, 1], 129, 1e-3, 1.0)
    assert n == 2
    assert math.isclose(out[0][0], 1.0 / (65 + 64 * math.exp(-50)), rel_tol=1e-14)


def check_locality(O):
    """gamma(t) >= k_e/k over multi-step trajectories with block fills."""
    rng = np.random.default_rng(25)
    d, G = 8, 2
    for k, k_e in ((8, 6), (6, 3), (5, 5)):
        T = 64 * 14 + 200
        keys = rng.standard_normal((T, d))
        vals = rng.standard_normal((T, d))
        logits = rng.standard_normal(T)
        row = O.OracleRow(keys, vals, logits, "f32", 0.3, k=k, k_e=k_e)
        L0 = 64 * 10 - 3
        for t in range(200):
            q = rng.standard_normal((G, d))
            res = row.step(L0 + t + 1, q, attend_out=False)
            if "gamma" in res:
                assert res["gamma"] >= k_e / k - 1e-15, (k, k_e, t, res["gamma"])
    # hand case: the previous selection and tail fully cover the new one
    assert O.locality([1, 2, 3], [1, 2], 3) == 1.0
    assert O.locality([1, 2, 4, 5], [1, 2, 3], None) == 0.5


# ----------------------------------------------------------------------------
# the multi-step driver: caches, state carried across steps, both modes
# ----------------------------------------------------------------------------
def _bf16_values(rng, shape):
    """Random values exactly representable in bf16 (torch's float32 -> bf16
    cast, a library routine independent of the oracle's rounding)."""
    import torch
    x = rng.standard_normal(shape).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()


def _expected_reps_and_E(keys, logits, nb):
    """Every block's representatives and eviction score from exact rationals."""
    d = keys.shape[1]
    reps = np.zeros((nb, 4, d))
    E = np.zeros(nb)
    for b in range(nb):
        means = []
        for j in range(4):
            lo = 64 * b + 16 * j
            for c in range(d):
                reps[b, j, c] = float(nearest_even_by_search(fsum_exact(keys[lo:lo + 16, c]) / 16, 8))
            means.append(fsum_exact(logits[lo:lo + 16]) / 16)
        E[b] = float(nearest_even_by_search(max(means), 24))
    return reps, E


def _loop_scores(q, reps, scale):
    """Group-softmax block scores written as loops over the stored reps."""
    nb, _, d = reps.shape
    G = len(q)
    group = [0.0] * (4 * nb)
    for h in range(G):
        lg = [scale * sum(q[h][c] * reps[j // 4, j % 4, c] for c in range(d)) for j in range(4 * nb)]
        mx = max(lg)
        z = sum(math.exp(v - mx) for v in lg)
        for j in range(4 * nb):
            group[j] += math.exp(lg[j] - mx) / z
    return [max(group[4 * b:4 * b + 4]) for b in range(nb)]


def _attend_tokens(q, keys, vals, toks, scale):
    out = np.zeros((len(q), keys.shape[1]))
    for h in range(len(q)):
        lg = [scale * float(np.dot(q[h], keys[t])) for t in toks]
        mx = max(lg)
        w = [math.exp(v - mx) for v in lg]
        z = sum(w)
        for i, t in enumerate(toks):
            out[h] += (w[i] / z) * vals[t]
    return out


def check_row_trajectory(O):
    """OracleRow over decode steps that fill blocks, in ascending and ordered
    mode.  At every step: its representatives and eviction scores (grown
    incrementally) equal exact-rational ones computed from scratch; the
    eviction set is the global top-k_e by E; the selection is the sort-based
    top of loop-computed scores; gamma is recomputed from the two selections
    and the previous tail; the output is attention over the selected tokens;
    in ordered mode the list is the sorted order and n* the brute-force prefix
    scan."""
    rng = np.random.default_rng(26)
    d, G, scale = 3, 2, 0.45
    nb_final = 9
    T = 64 * nb_final + 40
    keys = _bf16_values(rng, (T, d))
    vals = rng.standard_normal((T, d))
    logits = rng.standard_normal(T).astype(np.float32).astype(np.float64)
    want_reps, want_E = _expected_reps_and_E(keys, logits, nb_final)
    L0 = 64 * 4 + 50                       # blocks 4, 5, ... fill along the way
    steps = 64 * nb_final - L0 + 20

    for k, k_e in ((5, 3), (4, 4)):
        row = O.OracleRow(keys, vals, logits, "bf16", scale, k=k, k_e=k_e)
        prev_sel, prev_tail = None, None
        for t in range(0, steps, 3):       # several steps skipped: fills arrive in bulk too
            L = L0 + t + 1
            nb = L // 64
            q = rng.standard_normal((G, d))
            res = row.step(L, q)
            assert np.array_equal(row.reps(nb), want_reps[:nb]), ("reps", t)
            assert np.array_equal(row.eviction_scores(nb), want_E[:nb]), ("E", t)
            ev = sorted(sorted(range(nb), key=lambda i: (-want_E[i], i))[:k_e])
            assert res["evict_set"].tolist() == ev, ("evict", t)
            S = _loop_scores(q, want_reps[:nb], scale)
            rest = [i for i in range(nb) if i not in ev]
            qa = sorted(rest, key=lambda i: (-S[i], i))[:min(k - len(ev), len(rest))]
            sel = sorted(ev + qa)
            assert res["selected"].tolist() == sel, ("selected", t)
            toks = [t_ for b in sel for t_ in range(64 * b, 64 * b + 64)] + list(range(64 * nb, L))
            assert np.allclose(res["out"], _attend_tokens(q, keys, vals, toks, scale),
                               rtol=0, atol=1e-12), ("out", t)
            if prev_sel is not None:
                resident = set(prev_sel) | ({prev_tail} if prev_tail is not None else set())
                assert res["gamma"] == len(set(sel) & resident) / len(sel), ("gamma", t)
            else:
                assert "gamma" not in res
            prev_sel, prev_tail = sel, (nb if L % 64 else None)

    tau, cap = 0.2, 6
    row = O.OracleRow(keys, vals, logits, "bf16", scale, k=cap, ordered=True, tau=tau)
    fired = 0
    for t in range(0, steps, 5):
        L = L0 + t + 1
        nb = L // 64
        q = 1.5 * rng.standard_normal((G, d))
        res = row.step(L, q)
        assert np.array_equal(row.reps(nb), want_reps[:nb]), ("ordered reps", t)
        S = _loop_scores(q, want_reps[:nb], scale)
        order = sorted(range(nb), key=lambda i: (-S[i], i))[:cap]
        assert res["selected"].tolist() == order, ("ordered list", t)
        n = brute_stop_index(q, keys, order, L, tau, scale)
        assert res["n_star"] == n, ("n*", t)
        fired += n < len(order)
        toks = [t_ for b in order[:n] for t_ in range(64 * b, 64 * b + 64)] + list(range(64 * nb, L))
        assert np.allclose(res["out"], _attend_tokens(q, keys, vals, toks, scale),
                           rtol=0, atol=1e-12), ("ordered out", t)
    assert fired >= 10, fired        # the stop fires before the end of the list


def check_residency_diff(O):
    """Set differences against a bitmap walk over every block id, the
    identity gamma = 1 - |fetch|/|S| with the (separately pinned) locality,
    and |S| - |fetch| = |A| - |release| (both are |S and A|)."""
    rng = np.random.default_rng(27)
    for trial in range(200):
        nmax = int(rng.integers(1, 40))
        S = rng.choice(nmax, int(rng.integers(0, nmax + 1)), replace=False)
        P_ = rng.choice(nmax, int(rng.integers(0, nmax + 1)), replace=False)
        tail = int(rng.integers(0, nmax + 3)) if rng.random() < 0.7 else None
        fetch, release = O.residency_diff(S, P_, tail)
        inS = [False] * (nmax + 3)
        inA = [False] * (nmax + 3)
        for b in S:
            inS[int(b)] = True
        for b in P_:
            inA[int(b)] = True
        if tail is not None:
            inA[tail] = True
        want_f = [b for b in range(nmax + 3) if inS[b] and not inA[b]]
        want_r = [b for b in range(nmax + 3) if inA[b] and not inS[b]]
        assert fetch.tolist() == want_f and release.tolist() == want_r, trial
        nA = sum(inA)
        assert len(S) - len(fetch) == nA - len(release)
        if len(S):
            assert math.isclose(1 - len(fetch) / len(S), O.locality(S, P_, tail), rel_tol=0,
                                abs_tol=1e-15)
    # hand case: resident {1, 2} + tail 3; selected {2, 3, 4} -> fetch {4}, release {1}
    f, r = O.residency_diff([4, 2, 3], [2, 1], 3)
    assert f.tolist() == [4] and r.tolist() == [1]


ALL_CHECKS = [
    check_round, check_rne_fraction, check_rounded_means, check_reps_layout,
    check_eviction_scores, check_scores_bruteforce, check_scores_closed_forms,
    check_forecast, check_forecast_window, check_topk_exchange, check_selection_golden, check_select_bruteforce,
    check_eviction_incremental, check_dense_reduction, check_attend_loops,
    check_attention_bias, check_early_stop, check_locality, check_row_trajectory, check_residency_diff,
]
