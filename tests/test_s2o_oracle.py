"""The S2O prefill oracle against its pins, and planted mistakes in copies of
it that some pin must catch (CPU only)."""

import importlib.util
import os
import sys

import numpy as np
import pytest

from oracle import s2o_prefill as S
from tests import s2o_pins as P

PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "oracle", "s2o_prefill.py")


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(S)


def fresh():
    spec = importlib.util.spec_from_file_location("oracle.s2o_prefill_mutant", PATH)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    try:
        spec.loader.exec_module(mod)
    finally:
        del sys.modules[spec.name]
    return mod


def mut_history_ascending(M):
    orig = M.history_order

    def f(q_seg, keys, start, storage):
        o, s = orig(q_seg, keys, start, storage)
        return np.lexsort((np.arange(s.size), s)).astype(np.int64), s
    M.history_order = f


def mut_guide_includes_segment(M):
    orig = M.query_order

    def f(q_seg, keys, start, storage):
        return orig(q_seg, keys, min(start + len(q_seg), len(keys)), storage)
    M.query_order = f


def mut_rep_from_history_queries(M):
    def f(q_seg, keys, start, storage):
        rep = M.stored_mean(np.asarray(q_seg)[: max(1, len(q_seg) // 2)], storage, q_seg.shape[1])
        s = np.asarray(keys[:start], dtype=np.float64) @ rep
        return M.descending_order(s), s
    M.history_order = f


def mut_ties_to_later(M):
    def f(scores):
        scores = np.asarray(scores, dtype=np.float64)
        return np.lexsort((-np.arange(scores.size), -scores)).astype(np.int64)
    M.descending_order = f


def mut_mean_not_rounded(M):
    def f(rows, storage, width):
        rows = np.asarray(rows, dtype=np.float64).reshape(-1, width)
        return rows.mean(axis=0) if rows.shape[0] else np.zeros(width)
    M.stored_mean = f


def _tile_variant(M, own_excl_diag=False, a_before=False, any_query=False, drop_last=False,
                  no_scale=False):
    def f(q_rows, positions, keys, values, start, kv_perm, tau, scale):
        if no_scale:
            scale = 1.0
        q_rows = np.asarray(q_rows, dtype=np.float64)
        tiles = M.history_tiles(kv_perm)
        hist = np.asarray(kv_perm, dtype=np.int64)
        n = q_rows.shape[0]
        own = [np.arange(start, int(p) + (0 if own_excl_diag and p > start else 1))
               for p in positions]
        c = np.array([((keys[np.concatenate([own[i], hist])] @ q_rows[i]) * scale).max()
                      for i in range(n)])

        def mass(i, tok):
            if len(tok) == 0:
                return 0.0
            return float(np.exp((keys[tok] @ q_rows[i]) * scale - c[i]).sum())

        A = np.array([mass(i, own[i]) for i in range(n)])
        n_star = len(tiles)
        for t, tok in enumerate(tiles):
            Mv = np.array([mass(i, tok) for i in range(n)])
            if not a_before:
                A = A + Mv
            hit = np.any(Mv < tau * A) if any_query else np.all(Mv < tau * A)
            if a_before:
                A = A + Mv
            if hit:
                n_star = t if drop_last else t + 1
                break
        kept = np.concatenate(tiles[:n_star]) if n_star else np.zeros(0, dtype=np.int64)
        out = np.stack([M.attend_tokens(q_rows[i], keys, values,
                                        np.concatenate([own[i], kept]), scale) for i in range(n)])
        return n_star, out
    M.query_tile = f


MUTANTS = {
    "history order ascending": mut_history_ascending,
    "guide vector includes the segment's own keys": mut_guide_includes_segment,
    "representative query from half the segment": mut_rep_from_history_queries,
    "equal scores to the later position": mut_ties_to_later,
    "means not rounded to the storage format": mut_mean_not_rounded,
    "pass 1 without the diagonal": lambda M: _tile_variant(M, own_excl_diag=True),
    "accumulated mass without the current tile": lambda M: _tile_variant(M, a_before=True),
    "stop when any query is below tau": lambda M: _tile_variant(M, any_query=True),
    "stopping tile dropped": lambda M: _tile_variant(M, drop_last=True),
    "softmax scale dropped": lambda M: _tile_variant(M, no_scale=True),
}


def test_unmutated_copy_passes():
    M = fresh()
    for check in P.ALL_CHECKS:
        check(M)


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    M = fresh()
    MUTANTS[name](M)
    caught = []
    for check in P.ALL_CHECKS:
        try:
            check(M)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no pin catches: {name}"
