"""CPU oracle for S2O prefill attention (segment permutations, two passes,
monotone-gain early stop).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
never calls it, and it shares no code, table or helper with the GPU path.

Plain float64 NumPy, one (sequence, query head) at a time, written from the
S2O technical summary (gist.science, Italian):

* "1. Permutazione Online tramite Caricamento Guidato da Indici": the
  sequence is cut into segments; inside each segment the queries are ordered
  by a coarse importance score taken against one shared guide vector
  (Q_perm), and the history before the segment is ordered by its score
  against one representative query of the segment, under the causal mask
  (KV_perm).  Tiles are then gathered by index; nothing moves in memory.
* "2. Regola di Arresto Anticipato": the permuted history is walked in
  descending estimated importance, and the walk ends once a tile's marginal
  attention mass is below tau times the mass accumulated so far.
* "3. Implementazione del Kernel": a first pass attends densely and causally
  inside the segment and seeds the online-softmax state (m, l, acc); the
  second pass resumes from it over the permuted history with the early stop.

Readings taken where the page leaves a step open (each is listed with its
reason in the design notes):

* Segments are ``seg`` consecutive tokens (the last one may be shorter);
  queries and history keys are grouped in tiles of 64 (``TILE``).
* The guide vector of segment s is the mean key of its history
  [0, s*seg); a query's coarse importance is its dot product with it, i.e.
  its mean logit over the history (up to the scale).  Segment 0 has no
  history, a zero guide, and keeps its queries in order.
* The representative query of a segment is the mean of its queries.
* Both means are stored like every other vector (in the input format): the
  exact sum of the stored rows, divided by the count in float64, rounded once
  to the storage format.
* Orders are by descending score, equal scores in ascending index order.
* Query tile j of a segment is Q_perm[64j : 64j+64]; history tile n is
  KV_perm[64n : 64n+64].  All 64 queries of a tile walk the history
  together: the walk stops after the first history tile whose mass is below
  tau times the accumulated mass (this tile included) for every query of
  the query tile, and that tile is kept.  The pass-1 mass seeds the
  accumulated mass.  Without such a tile the whole history is attended;
  tau = 0 therefore gives dense causal attention.
* Each query head is its own problem (its KV head is h // G); the history
  order is per query head.
"""

from __future__ import annotations

import math

import numpy as np

from .nsa_oracle import round_storage

TILE = 64


def segment_bounds(L: int, seg: int):
    """[(start, end)] of the segments of a sequence of L tokens."""
    return [(s, min(s + seg, L)) for s in range(0, L, seg)]


def stored_mean(rows: np.ndarray, storage: str, width: int) -> np.ndarray:
    """Mean of stored rows as a stored vector: the exact column sums
    (``math.fsum``), divided by the row count in float64, rounded once to the
    storage format.  No rows: the zero vector."""
    rows = np.asarray(rows, dtype=np.float64).reshape(-1, width)
    n = rows.shape[0]
    if n == 0:
        return np.zeros(width)
    sums = np.array([math.fsum(rows[:, c]) for c in range(width)])
    return round_storage(sums / n, storage)


def descending_order(scores: np.ndarray) -> np.ndarray:
    """Positions sorted by descending score, equal scores by ascending position."""
    scores = np.asarray(scores, dtype=np.float64)
    return np.lexsort((np.arange(scores.size), -scores)).astype(np.int64)


def query_order(q_seg: np.ndarray, keys: np.ndarray, start: int, storage: str):
    """Q_perm of the segment starting at ``start``: offsets inside the segment
    by descending importance against the guide vector (the stored mean key
    of tokens [0, start)).  Returns (order, scores)."""
    d = q_seg.shape[1]
    guide = stored_mean(keys[:start], storage, d)
    s = np.asarray(q_seg, dtype=np.float64) @ guide
    return descending_order(s), s


def history_order(q_seg: np.ndarray, keys: np.ndarray, start: int, storage: str):
    """KV_perm of the segment starting at ``start``: the history tokens
    [0, start) by descending score against the representative query (the
    stored mean of the segment's queries).  Returns (order, scores)."""
    d = q_seg.shape[1]
    rep = stored_mean(q_seg, storage, d)
    s = np.asarray(keys[:start], dtype=np.float64) @ rep
    return descending_order(s), s


def history_tiles(kv_perm: np.ndarray):
    return [np.asarray(kv_perm[i:i + TILE], dtype=np.int64) for i in range(0, len(kv_perm), TILE)]


def attend_tokens(q: np.ndarray, keys: np.ndarray, values: np.ndarray, tokens, scale: float):
    """softmax(q . k_t * scale) over ``tokens``, applied to V (two-pass, fp64)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    lg = (keys[tokens] @ np.asarray(q, dtype=np.float64)) * scale
    w = np.exp(lg - lg.max())
    return (w / w.sum()) @ values[tokens]


def query_tile(q_rows, positions, keys, values, start: int, kv_perm, tau: float, scale: float):
    """Both passes for one tile of permuted queries.  Returns (n_star, out).

    q_rows: [n][d] the tile's queries; positions: their token positions.
    Pass 1 (dense, causal, inside the segment): query at position p sees
    tokens [start, p].  Pass 2: history tiles in KV_perm order; M_i(n) and
    A_i(n) are query i's mass of tile n and its accumulated mass including
    tile n, both relative to one common shift c_i (it cancels in the ratio).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    tiles = history_tiles(kv_perm)
    hist = np.asarray(kv_perm, dtype=np.int64)
    n = q_rows.shape[0]
    own = [np.arange(start, int(p) + 1) for p in positions]
    c = np.empty(n)
    for i in range(n):
        reach = np.concatenate([own[i], hist])
        c[i] = ((keys[reach] @ q_rows[i]) * scale).max()

    def mass(i, tok):
        if len(tok) == 0:
            return 0.0
        return float(np.exp((keys[tok] @ q_rows[i]) * scale - c[i]).sum())

    A = np.array([mass(i, own[i]) for i in range(n)])
    n_star = len(tiles)
    for t, tok in enumerate(tiles):
        M = np.array([mass(i, tok) for i in range(n)])
        A = A + M
        if np.all(M < tau * A):
            n_star = t + 1
            break
    kept = np.concatenate(tiles[:n_star]) if n_star else np.zeros(0, dtype=np.int64)
    out = np.stack([attend_tokens(q_rows[i], keys, values, np.concatenate([own[i], kept]), scale)
                    for i in range(n)])
    return n_star, out


def prefill_head(q, keys, values, seg: int, tau: float, scale: float, storage: str,
                 q_perms=None, kv_perms=None):
    """S2O prefill of one query head over a sequence of L = len(q) tokens.

    q: [L][d] the head's queries; keys, values: [L][d] its KV head's tokens
    (all widened exactly to float64).  q_perms / kv_perms: optional per-segment
    orders to use instead of computing them (to evaluate the attention on an
    order produced elsewhere).  Returns a dict with the per-segment orders and
    scores, n_star per (segment, query tile), and out [L][d].
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    L, d = q.shape
    res = {"q_perm": [], "kv_perm": [], "q_score": [], "kv_score": [], "n_star": [],
           "out": np.zeros((L, d))}
    for s, (a, b) in enumerate(segment_bounds(L, seg)):
        q_seg = q[a:b]
        qo, qs = query_order(q_seg, keys, a, storage)
        ko, ks = history_order(q_seg, keys, a, storage)
        if q_perms is not None:
            qo = np.asarray(q_perms[s], dtype=np.int64)
        if kv_perms is not None:
            ko = np.asarray(kv_perms[s], dtype=np.int64)
        res["q_perm"].append(qo)
        res["kv_perm"].append(ko)
        res["q_score"].append(qs)
        res["kv_score"].append(ks)
        stars = []
        for j in range(0, b - a, TILE):
            offs = qo[j:j + TILE]
            pos = a + offs
            n_star, out = query_tile(q[pos], pos, keys, values, a, ko, tau, scale)
            res["out"][pos] = out
            stars.append(n_star)
        res["n_star"].append(stars)
    return res
