"""Plant a mistake in a copy of the oracle; some pin must catch it.

This shows the pins are sharp enough: a dropped term, a wrong index, a
reversed tie rule or a lost token would not slip through.
"""

import importlib.util
import os
import sys

import numpy as np
import pytest

from tests import oracle_pins as P

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "oracle", "nsa_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("nsa_oracle_mutant", ORACLE_PATH)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod          # dataclasses look the module up by name
    try:
        spec.loader.exec_module(mod)
    finally:
        del sys.modules[spec.name]
    return mod


def mut_no_softmax(O):
    def f(q, reps, scale):
        nb, nsub, d = reps.shape
        lg = (np.asarray(q) @ reps.reshape(nb * nsub, d).T) * scale
        return lg.sum(axis=0).reshape(nb, nsub).max(axis=1)
    O.block_scores_group_softmax = f


def mut_max_before_head_sum(O):
    def f(q, reps, scale):
        nb, nsub, d = reps.shape
        lg = (np.asarray(q) @ reps.reshape(nb * nsub, d).T) * scale
        p = np.exp(lg - lg.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        return p.reshape(len(q), nb, nsub).max(axis=2).sum(axis=0)
    O.block_scores_group_softmax = f


def mut_ties_to_higher_id(O):
    def f(ids, scores, k):
        ids = np.asarray(ids, dtype=np.int64)
        order = np.lexsort((-ids, -np.asarray(scores, dtype=np.float64)))
        return ids[order[:k]]
    O.top_k = f


def mut_tail_dropped(O):
    def f(blocks, L):
        parts = [np.arange(b * 64, (b + 1) * 64) for b in blocks] + [np.zeros(0, dtype=np.int64)]
        return np.concatenate(parts).astype(np.int64)
    O.token_set = f


def mut_stop_block_excluded(O):
    orig = O.early_stop_attention

    def f(q, keys, values, order, L, tau, scale, bias=None):
        n, _ = orig(q, keys, values, order, L, tau, scale, bias)
        n2 = n - 1 if n < len(order) else n
        return n2, O.sparse_attention(q, keys, values, list(order[:n2]), L, scale, bias)
    O.early_stop_attention = f


def mut_sub_block_shift(O):
    def f(keys, nb, storage):
        d = keys.shape[1]
        x = np.asarray(keys[1: nb * 64 + 1], dtype=np.float64).reshape(nb, 4, 16, d)
        return O.rounded_means(np.moveaxis(x, 2, 3), storage)
    O.block_reps = f


def mut_eviction_forgets_old(O):
    def f(prev_set, n_seen, nb, E, k_e):
        cand = np.arange(n_seen, nb, dtype=np.int64)
        if k_e == 0 or cand.size == 0:
            return np.asarray(prev_set, dtype=np.int64)
        return np.sort(O.top_k(cand, E[cand], min(k_e, cand.size)))
    O.eviction_update = f


def mut_attention_unscaled(O):
    orig = O.attend
    O.attend = lambda q, K, V, scale, bias=None: orig(q, K, V, 1.0, bias)


def mut_round_truncates(O):
    def f(x):
        x = np.asarray(x, dtype=np.float64)
        m, e = np.frexp(x)
        return np.ldexp(np.trunc(m * 256.0) / 256.0, e)
    O.round_bf16 = f


def mut_parts_overlap(O):
    def f(S, evict_set, nb, k):
        return O.top_k(np.arange(nb), S, min(k - len(evict_set), nb))
    O.query_aware_set = f


def mut_mean_by_15(O):
    orig = O.rounded_means
    O.rounded_means = lambda x, storage: orig(np.asarray(x) * (16.0 / 15.0), storage)


def mut_gamma_ignores_tail(O):
    def f(selected, prev_selected, prev_tail_block):
        sel = set(int(b) for b in selected)
        return len(sel & set(int(b) for b in prev_selected)) / max(len(sel), 1)
    O.locality = f


def mut_row_reps_from_previous_block(O):
    """The incremental representatives extend from block n0 - 1 instead of n0."""
    def reps(self, nb):
        if self._reps.shape[0] < nb:
            n0 = self._reps.shape[0]
            new = O.block_reps(self.keys[max(n0 - 1, 0) * 64:], nb - n0, self.storage)
            self._reps = np.concatenate([self._reps, new])
        return self._reps[:nb]
    O.OracleRow.reps = reps


def mut_row_eviction_from_previous_block(O):
    """The incremental eviction scores extend from block n0 - 1 instead of n0."""
    def eviction_scores(self, nb):
        if self._E.shape[0] < nb:
            n0 = self._E.shape[0]
            new = O.eviction_block_scores(self.logits[max(n0 - 1, 0) * 64:], nb - n0)
            self._E = np.concatenate([self._E, new])
        return self._E[:nb]
    O.OracleRow.eviction_scores = eviction_scores


def mut_row_prev_tail_off_by_one(O):
    """The step records the block before the tail as the previous tail."""
    orig = O.OracleRow.step

    def step(self, L, q, f=None, attend_out=True):
        res = orig(self, L, q, f=f, attend_out=attend_out)
        if self.state.prev_tail_block is not None:
            self.state.prev_tail_block -= 1
        return res
    O.OracleRow.step = step


def mut_row_ordered_stop_ignored(O):
    """The ordered branch attends the whole list (no early stop)."""
    orig = O.early_stop_attention

    def f(q, keys, values, order, L, tau, scale):
        return orig(q, keys, values, order, L, 0.0, scale)
    orig_step = O.OracleRow.step

    def step(self, L, q, f_=None, attend_out=True, **kw):
        if self.ordered:
            saved = O.early_stop_attention
            O.early_stop_attention = f
            try:
                return orig_step(self, L, q, attend_out=attend_out, **kw)
            finally:
                O.early_stop_attention = saved
        return orig_step(self, L, q, f_, attend_out=attend_out, **kw)
    O.OracleRow.step = step


def mut_residency_ignores_tail(O):
    """The previous step's tail block is not counted as resident."""
    orig = O.residency_diff
    O.residency_diff = lambda sel, prev, tail: orig(sel, prev, None)


def mut_residency_swapped(O):
    """Fetch and release swapped."""
    orig = O.residency_diff

    def f(sel, prev, tail):
        a, b = orig(sel, prev, tail)
        return b, a
    O.residency_diff = f


def mut_window_across_blocks(O):
    """A block also owns the window that reaches into the next block."""
    def f(fv, reps):
        nb, nsub, d = reps.shape
        flat = reps.reshape(nb * nsub, d)
        nxt = np.concatenate([flat[1:], flat[-1:]], axis=0)
        s = ((flat + nxt) / 2.0) @ np.asarray(fv, dtype=np.float64)
        return s.reshape(nb, nsub).max(axis=1)
    O.block_scores_forecast_window = f


def mut_window_skips_a_sub_block(O):
    """A window pairs sub-blocks j and j + 2."""
    def f(fv, reps):
        w = (reps[:, :-2, :] + reps[:, 2:, :]) / 2.0
        nb, n, d = w.shape
        return (w.reshape(nb * n, d) @ np.asarray(fv, dtype=np.float64)).reshape(nb, n).max(axis=1)
    O.block_scores_forecast_window = f


def mut_bias_subtracted(O):
    """The eviction logit lowers the token's weight instead of raising it."""
    orig = O.attend

    def f(q, K, V, scale, bias=None):
        return orig(q, K, V, scale, None if bias is None else -np.asarray(bias))
    O.attend = f


def mut_bias_missing_from_stop_masses(O):
    """The early-stop masses leave the bias out (the output keeps it)."""
    orig = O.early_stop_attention

    def f(q, keys, values, order, L, tau, scale, bias=None):
        n, _ = orig(q, keys, values, order, L, tau, scale)
        return n, O.sparse_attention(q, keys, values, list(order[:n]), L, scale, bias)
    O.early_stop_attention = f


MUTANTS = [mut_no_softmax, mut_max_before_head_sum, mut_ties_to_higher_id, mut_tail_dropped,
           mut_stop_block_excluded, mut_sub_block_shift, mut_eviction_forgets_old,
           mut_attention_unscaled, mut_round_truncates, mut_parts_overlap, mut_mean_by_15,
           mut_gamma_ignores_tail, mut_row_reps_from_previous_block,
           mut_row_eviction_from_previous_block, mut_row_prev_tail_off_by_one,
           mut_row_ordered_stop_ignored, mut_residency_ignores_tail,
           mut_residency_swapped, mut_window_across_blocks, mut_window_skips_a_sub_block,
           mut_bias_subtracted, mut_bias_missing_from_stop_masses]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_mutant_is_caught(mutant):
    O = fresh_oracle()
    mutant(O)
    caught = []
    for check in P.ALL_CHECKS:
        try:
            check(O)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no pin catches {mutant.__name__}"
