"""CPU oracle for block-sparse long-context decode attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
never calls it, and it shares no code, table or helper with the GPU path.

Plain float64 NumPy, one row at a time (a row is one sequence b and one KV
head g with its G query heads), written step by step from the pages:

* NOSA technical summary (gist.science, Spanish), "Metodología / 1. Algoritmo:
  NOSA": two-part selection (a query-aware part and a query-agnostic eviction
  part with a fixed budget k_e), the strict eviction rule, the locality bound
  gamma(t) >= k_e/k, block-granular selection scored by two-stage pooling
  (mean inside sub-blocks, then the maximum over a block), and selection on
  pre-exponential eviction scores (ED-DMA).
* SparDA technical summary (gist.science, German), "2. Methodik /
  Kompakter Forecast-Indexer": one forecast vector per KV head (GQA group),
  no per-query-head loop and no softmax in the selector; "Trainingsstrategie":
  the inference window of 32 tokens with stride 16.
* S2O technical summary (gist.science, Italian), "2. Regola di Arresto
  Anticipato" and "3. Implementazione del Kernel": blocks walked in descending
  estimated importance, stop once the marginal attention mass of a block is
  below tau times the accumulated mass; a first dense pass seeds the online
  softmax state.

Where the pages leave a step open, the reading taken is stated at the function
that implements it.  Every function here is pinned by ``tests/test_oracle_*``
against brute force, closed forms, library routines or hand-worked fixtures;
none is "parity unpinned".  The *readings* themselves (which score the pages
mean) are choices, listed with their reasons in the design notes.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from fractions import Fraction

import numpy as np

BLOCK = 64      # tokens per block
SUB = 16        # tokens per sub-block (4 sub-blocks per block)


# =============================================================================
# Storage rounding (the representative of a sub-block is one rounding of its
# exact mean to the storage format)
# =============================================================================
def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits.  ``frexp`` writes x = m * 2**e with
    0.5 <= |m| < 1, so m*256 carries exactly the 8 bits to keep and ``rint``
    (round half to even) rounds the rest away in one step.  Values below the
    bf16 normal range are outside the contract (no subnormal handling).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def round_f32(x) -> np.ndarray:
    """Round float64 values to the nearest float32 value, ties to even."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_storage(x, storage: str) -> np.ndarray:
    if storage == "bf16":
        return round_bf16(x)
    if storage == "f32":
        return round_f32(x)
    raise ValueError(storage)


def rne_fraction(q: Fraction, bits: int) -> Fraction:
    """Round an exact rational to ``bits`` significant bits, ties to even."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2**e <= a < 2**(e+1)
    unit = Fraction(2) ** (e - bits + 1)
    scaled = a / unit
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * unit


_BITS = {"bf16": 8, "f32": 24}


def rounded_means(x: np.ndarray, storage: str) -> np.ndarray:
    """One storage rounding of the exact mean over the last axis.

    The sum runs in float64 in index order; every addition is checked with
    Knuth's TwoSum (the rounding error of a+b is exactly recoverable).  Where
    all additions were exact, the float64 sum is the exact sum and dividing
    by the (power of two) count is exact, so one rounding follows.  Any entry
    with an inexact addition is recomputed with exact rationals and rounded
    directly from the rational value.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    total = x[..., 0].copy()
    exact = np.ones(total.shape, dtype=bool)
    for i in range(1, n):
        a, b = total, x[..., i]
        s = a + b
        bb = s - a
        err = (a - (s - bb)) + (b - bb)
        exact &= err == 0
        total = s
    assert n & (n - 1) == 0, "count must be a power of two"
    out = round_storage(total / n, storage)
    if not exact.all():
        bits = _BITS[storage]
        for idx in zip(*np.nonzero(~exact)):
            q = sum((Fraction(float(v)) for v in x[idx]), Fraction(0)) / n
            out[idx] = float(rne_fraction(q, bits))
    return out


# =============================================================================
# Step 1: block representatives
# =============================================================================
def block_reps(keys: np.ndarray, nb: int, storage: str) -> np.ndarray:
    """Sub-block mean keys of the first ``nb`` full blocks: [nb][4][d].

    NOSA summary, "Implementación Basada en Bloques": selection works on
    blocks of tokens, and the first pooling stage is a mean inside each
    sub-block.  By linearity the mean of the per-token scores q.k_t over a
    sub-block equals q.(mean of k_t), so the mean key is the representative.
    Reading: stored in the KV dtype as one round-to-nearest-even rounding of
    the exact mean.
    """
    d = keys.shape[1]
    x = np.asarray(keys[: nb * BLOCK], dtype=np.float64).reshape(nb, BLOCK // SUB, SUB, d)
    return rounded_means(np.moveaxis(x, 2, 3), storage)          # [nb][4][d]


def eviction_block_scores(logits: np.ndarray, nb: int) -> np.ndarray:
    """Query-agnostic block scores E: [nb] (values representable in float32).

    NOSA summary, "Mecanismo de Doble Selección" and "ED-DMA": an eviction
    head gives every token a query-independent score and selection ranks on
    the pre-exponential score.  Reading: the per-token logits are inputs, and
    E pools them with the same two stages (sub-block mean, block maximum),
    rounded once to float32.  Rounding is monotone, so the maximum of the
    rounded means is the rounding of the maximum of the exact means.
    """
    x = np.asarray(logits[: nb * BLOCK], dtype=np.float64).reshape(nb, BLOCK // SUB, SUB)
    return rounded_means(x, "f32").max(axis=1)


# =============================================================================
# Step 2: block scores
# =============================================================================
def block_scores_group_softmax(q: np.ndarray, reps: np.ndarray, scale: float) -> np.ndarray:
    """NOSA-mode block scores S: [nb].

    For each query head h of the group: logits (q_h . r_j) * scale over every
    sub-block j of the row, softmax over j; the group's sub-block score is
    the sum of the heads' probabilities; a block scores the maximum over its
    4 sub-blocks (NOSA summary, "Implementación Basada en Bloques").
    Readings: the selector normalises per head with a softmax (the SparDA
    summary, "Kompakter Forecast-Indexer", names the softmax and the per-head
    loop as the cost its forecast removes); heads are summed before the
    block maximum.
    """
    nb, nsub, d = reps.shape
    if nb == 0:                       # no full block yet: nothing to score
        return np.zeros(0)
    r = reps.reshape(nb * nsub, d)
    logits = (np.asarray(q, dtype=np.float64) @ r.T) * scale            # [G][4nb]
    logits = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p = p / p.sum(axis=1, keepdims=True)
    group = p.sum(axis=0)                                               # [4nb]
    return group.reshape(nb, nsub).max(axis=1)


def block_scores_forecast(f: np.ndarray, reps: np.ndarray) -> np.ndarray:
    """SparDA-mode block scores S: [nb] -- raw f . r_j, maximum over the block.

    SparDA summary, "Kompakter Forecast-Indexer": one forecast vector per KV
    head, no per-query-head loop, no softmax.  Reading: no 1/sqrt(d) scale
    (it cannot change the ranking).
    """
    nb, nsub, d = reps.shape
    s = reps.reshape(nb * nsub, d) @ np.asarray(f, dtype=np.float64)
    return s.reshape(nb, nsub).max(axis=1)


def block_scores_forecast_window(f: np.ndarray, reps: np.ndarray) -> np.ndarray:
    """SparDA inference-window block scores S: [nb] -- raw f . w, maximum over
    the windows of a block.

    SparDA summary, "Trainingsstrategie": the selector's inference grid is a
    compression window of 32 tokens with stride 16.  The window that starts
    at a sub-block boundary covers two adjacent 16-token sub-blocks, so its
    mean is the mean of their two means, w = (r_j + r_{j+1}) / 2.  Readings:
    a block owns the three windows that lie inside it (starting at its tokens
    0, 16 and 32; the window starting at token 48 reaches into the next block
    and belongs to neither), its score is the largest f . w over them, and,
    as in the raw forecast mode, there is no scale and no softmax.
    """
    nb, nsub, d = reps.shape
    w = (reps[:, :-1, :] + reps[:, 1:, :]) / 2.0                 # [nb, nsub - 1, d]
    s = w.reshape(nb * (nsub - 1), d) @ np.asarray(f, dtype=np.float64)
    return s.reshape(nb, nsub - 1).max(axis=1)


# =============================================================================
# Step 3: selection
# =============================================================================
def top_k(ids: np.ndarray, scores: np.ndarray, k: int) -> np.ndarray:
    """The k best ids by descending score; equal scores go to the lower id.

    Returns them best first.
    """
    ids = np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -np.asarray(scores, dtype=np.float64)))
    return ids[order[:k]]


def eviction_update(prev_set: np.ndarray, n_seen: int, nb: int, E: np.ndarray,
                    k_e: int) -> np.ndarray:
    """Query-agnostic eviction set after the blocks [n_seen, nb) became full.

    NOSA summary, "Mecanismo de Doble Selección": content the eviction part
    drops at one step can never be picked by it again.  Reading: the
    candidates are the previous set plus the newly full blocks; the k_e best
    by E (ties to the lower id) survive.  Returned ascending.
    """
    cand = np.concatenate([np.asarray(prev_set, dtype=np.int64),
                           np.arange(n_seen, nb, dtype=np.int64)])
    if k_e == 0 or cand.size == 0:
        return np.zeros(0, dtype=np.int64)
    keep = top_k(cand, E[cand], min(k_e, cand.size))
    return np.sort(keep)


def query_aware_set(S: np.ndarray, evict_set: np.ndarray, nb: int, k: int) -> np.ndarray:
    """Query-aware part: the best k - |evict_set| blocks outside the eviction set.

    NOSA summary, "Mecanismo de Doble Selección": the query picks specific,
    possibly distant blocks, including ones the eviction part dropped.
    Reading: the two parts are disjoint, so k blocks are chosen when nb >= k.
    """
    rest = np.setdiff1d(np.arange(nb, dtype=np.int64), evict_set)
    m = min(k - len(evict_set), rest.size)
    return top_k(rest, S[rest], m)


def select_blocks(S: np.ndarray, evict_set: np.ndarray, nb: int, k: int) -> np.ndarray:
    """Selected blocks, ascending: eviction set plus query-aware set."""
    return np.sort(np.concatenate([np.asarray(evict_set, dtype=np.int64),
                                   query_aware_set(S, evict_set, nb, k)]))


def select_ordered(S: np.ndarray, nb: int, cap: int) -> np.ndarray:
    """Early-stop mode: the best ``cap`` blocks by descending score (ties: lower id).

    S2O summary, "2. Regola di Arresto Anticipato": candidate blocks are
    processed in descending estimated importance.
    """
    return top_k(np.arange(nb, dtype=np.int64), S, min(cap, nb))


# =============================================================================
# Step 4: attention over the selected blocks and the partial tail block
# =============================================================================
def token_set(blocks, L: int) -> np.ndarray:
    """Token ids of the given full blocks followed by the partial tail block.

    Reading: the current token is appended first and then attended; the
    partial last block (tokens [64*floor(L/64), L)) is always attended and is
    never scored or counted in k.
    """
    nb = L // BLOCK
    parts = [np.arange(b * BLOCK, (b + 1) * BLOCK) for b in blocks]
    parts.append(np.arange(nb * BLOCK, L))
    return np.concatenate(parts).astype(np.int64)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, bias=None) -> np.ndarray:
    """softmax((q . k_t) * scale [+ bias_t]) over the given tokens, applied to
    V: [G][d].

    Plain two-pass softmax in float64.  bias: one additive logit per token
    (the eviction logit under the ED-DMA reading, see sparse_attention), or
    None.
    """
    logits = (np.asarray(q, dtype=np.float64) @ np.asarray(K, dtype=np.float64).T) * scale
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    logits = logits - logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ np.asarray(V, dtype=np.float64)


def sparse_attention(q, keys, values, blocks, L: int, scale: float, bias=None) -> np.ndarray:
    """Attention over the given blocks plus the partial tail block.

    bias (optional): the row's per-token eviction logits e_t in logical
    token order.  NOSA summary, "ED-DMA": the eviction head selects on
    pre-exponential scores and its exponential is deferred to the attention
    stage.  Reading (a variant, off by default): exp(e_t) weights token t
    inside the attention softmax, i.e. e_t is added to its logit.
    """
    t = token_set(blocks, L)
    return attend(q, keys[t], values[t], scale, None if bias is None else np.asarray(bias)[t])


def early_stop_attention(q, keys, values, order, L: int, tau: float, scale: float, bias=None):
    """Ordered traversal with the monotone-gain early stop.  Returns (n_star, out).

    S2O summary, "2. Regola di Arresto Anticipato" and "3. Implementazione del
    Kernel": the partial tail block is attended first and seeds the
    accumulated mass; then blocks pi_1, pi_2, ... are taken in the given
    order.  Readings: the mass of block n for head h is
    M_h(n) = sum over its tokens of exp(logit - c) (c is any common shift; it
    cancels in the ratio), the accumulated mass A_h(n) includes block n, and
    the walk stops after the first block with M_h(n) < tau * A_h(n) for
    every head of the group (the block is loaded once for all of them); that
    block is kept.  Without such a block every listed block is attended.
    With the ED-DMA bias (see sparse_attention) a token's logit includes its
    eviction logit, in the masses as in the output.
    """
    q = np.asarray(q, dtype=np.float64)
    nb = L // BLOCK
    tail = np.arange(nb * BLOCK, L)
    blocks = [np.arange(b * BLOCK, (b + 1) * BLOCK) for b in order]
    every = np.concatenate([tail] + blocks).astype(np.int64)
    e = np.zeros(keys.shape[0]) if bias is None else np.asarray(bias, dtype=np.float64)
    logits_all = (q @ keys[every].T) * scale + e[every][None, :]
    c = logits_all.max(axis=1, keepdims=True)

    def mass(tok):
        if tok.size == 0:
            return np.zeros(q.shape[0])
        return np.exp((q @ keys[tok].T) * scale + e[tok][None, :] - c).sum(axis=1)

    A = mass(tail)
    n_star = len(order)
    for n, tok in enumerate(blocks, start=1):
        M = mass(tok)
        A = A + M
        if np.all(M < tau * A):
            n_star = n
            break
    out = sparse_attention(q, keys, values, list(order[:n_star]), L, scale, bias)
    return n_star, out


# =============================================================================
# Locality bookkeeping
# =============================================================================
def locality(selected, prev_selected, prev_tail_block) -> float:
    """gamma(t): the fraction of this step's blocks that were resident at t-1.

    NOSA summary, "Garantía de Localidad".  Reading: resident at t-1 means
    selected at t-1 or being the partial tail block then (it was attended).
    """
    sel = set(int(b) for b in selected)
    if not sel:
        return 1.0
    resident = set(int(b) for b in prev_selected)
    if prev_tail_block is not None:
        resident.add(int(prev_tail_block))
    return len(sel & resident) / len(sel)


def residency_diff(selected, prev_selected, prev_tail_block):
    """Blocks to fetch and to release between consecutive steps: (fetch, release).

    NOSA summary, "2. Sistema: NOSI": with the cache kept in block units, a
    step moves only what its selection adds to, or drops from, the blocks
    already in place; "Garantía de Localidad" bounds how much that is.
    Reading: the resident set after step t-1 is its selection plus its
    partial tail block (attended then); fetch = S_t minus that set, release =
    that set minus S_t, both ascending.  1 - |fetch|/|S_t| is gamma(t).
    """
    S = np.unique(np.asarray(selected, dtype=np.int64))
    A = np.asarray(prev_selected, dtype=np.int64)
    if prev_tail_block is not None:
        A = np.concatenate([A, np.array([prev_tail_block], dtype=np.int64)])
    A = np.unique(A)
    return np.setdiff1d(S, A), np.setdiff1d(A, S)


# =============================================================================
# One decode step of one row, with the state that crosses steps
# =============================================================================
@dataclass
class RowState:
    evict_set: np.ndarray = field(default_factory=lambda: np.zeros(0, dtype=np.int64))
    n_seen: int = 0
    prev_selected: np.ndarray | None = None
    prev_tail_block: int | None = None


class OracleRow:
    """A row's cache (stored values widened to float64) and its selection state.

    ``keys``/``values`` [T][d] and ``logits`` [T] hold every token the row
    will ever have; a step only looks at the first L of them.
    """

    def __init__(self, keys, values, logits, storage: str, scale: float,
                 mode: str = "group_softmax", k: int = 16, k_e: int = 0,
                 ordered: bool = False, tau: float = 0.0):
        self.keys = np.asarray(keys, dtype=np.float64)
        self.values = np.asarray(values, dtype=np.float64)
        self.logits = None if logits is None else np.asarray(logits, dtype=np.float64)
        self.storage, self.scale, self.mode = storage, scale, mode
        self.k, self.k_e, self.ordered, self.tau = k, k_e, ordered, tau
        self.state = RowState()
        self._reps = np.zeros((0, BLOCK // SUB, self.keys.shape[1]))
        self._E = np.zeros(0)

    def reps(self, nb: int) -> np.ndarray:
        if self._reps.shape[0] < nb:
            n0 = self._reps.shape[0]
            new = block_reps(self.keys[n0 * BLOCK:], nb - n0, self.storage)
            self._reps = np.concatenate([self._reps, new])
        return self._reps[:nb]

    def eviction_scores(self, nb: int) -> np.ndarray:
        if self._E.shape[0] < nb:
            n0 = self._E.shape[0]
            new = eviction_block_scores(self.logits[n0 * BLOCK:], nb - n0)
            self._E = np.concatenate([self._E, new])
        return self._E[:nb]

    def scores(self, nb: int, q=None, f=None) -> np.ndarray:
        if self.mode == "forecast":
            return block_scores_forecast(f, self.reps(nb))
        if self.mode == "forecast_window":
            return block_scores_forecast_window(f, self.reps(nb))
        return block_scores_group_softmax(q, self.reps(nb), self.scale)

    def step(self, L: int, q, f=None, attend_out: bool = True) -> dict:
        """Decode step with L cached tokens (the current one included)."""
        nb = L // BLOCK
        st = self.state
        S = self.scores(nb, q=q, f=f)
        res = {"L": L, "nb": nb, "S": S}
        if self.ordered:
            order = select_ordered(S, nb, self.k)
            res["selected"] = order
            if attend_out:
                n_star, out = early_stop_attention(q, self.keys, self.values, order, L,
                                                   self.tau, self.scale)
                res["n_star"], res["out"] = n_star, out
            return res
        if self.k_e > 0:
            E = self.eviction_scores(nb)
            evict = eviction_update(st.evict_set, st.n_seen, nb, E, self.k_e)
            res["E"] = E
        else:
            evict = np.zeros(0, dtype=np.int64)
        sel = select_blocks(S, evict, nb, self.k)
        res["evict_set"], res["selected"] = evict, sel
        if st.prev_selected is not None:
            res["gamma"] = locality(sel, st.prev_selected, st.prev_tail_block)
        if attend_out:
            res["out"] = sparse_attention(q, self.keys, self.values, sel, L, self.scale)
        st.evict_set, st.n_seen = evict, nb
        st.prev_selected = sel
        st.prev_tail_block = nb if L % BLOCK else None
        return res


def dense_attention(q, keys, values, L: int, scale: float) -> np.ndarray:
    """Attention over all L cached tokens (the reference that k = all reduces to)."""
    return attend(q, keys[:L], values[:L], scale)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
