"""CPU checks of the fused step's launch geometry (nsa_decode_step_grid):
the invariants its waits rest on, over a sweep of shapes and device
capacities.  No kernel is launched.

* the grid never exceeds the resident capacity, so on an otherwise idle
  device every scorer runs at the same time as the other scorers of its
  gang (a scorer waits only on those, and on its gang's partials);
* the scorers hold every representative of the longest row;
* gangs have at most 64 members, attenders only where an eviction set
  exists and at most one per eviction item;
* the block-index rule (scorers of all gangs first, then attenders) maps
  the grid one-to-one onto (role, gang, member).
"""

from __future__ import annotations

import itertools
import math

import pytest

N = pytest.importorskip("block_sparse_kv_nsa_amd")


def grid_for(B, Hq, Hkv, D, dtype, k, k_e, L, cap, mode=0):
    mb = math.ceil(L / 64) + 1
    shape = N.Shape.make(B, Hq, Hkv, D, mb, B * mb, dtype)
    return N.nsa_decode_step_grid(shape, N.SelectParams(mode, k, k_e, 0), L, cap)


CASES = list(itertools.product(
    [(4, 32, 8, 128, N.NSA_BF16), (8, 16, 2, 128, N.NSA_BF16), (32, 32, 8, 128, N.NSA_BF16),
     (1, 4, 1, 64, N.NSA_F32), (3, 16, 2, 128, N.NSA_F32), (2, 16, 2, 64, N.NSA_BF16)],
    [(64, 48), (32, 0), (16, 8), (8, 8)],
    [100, 64 * 41 + 37, 16384 + 1, 131072 + 1, 64 * 2600 + 11],
    [256, 512, 100, 13]))


@pytest.mark.parametrize("geom,sel,L,cap", CASES)
def test_plan_invariants(geom, sel, L, cap):
    B, Hq, Hkv, D, dtype = geom
    k, k_e = sel
    rows = B * Hkv
    nsub = 4 * (L // 64)
    G = Hq // Hkv
    reps_cap = 512 if (dtype == N.NSA_F32 and D == 128 and G == 8) else 1024
    try:
        g = grid_for(B, Hq, Hkv, D, dtype, k, k_e, L, cap)
    except N.NsaError as e:
        # only when not even one gang of the needed scorers fits
        assert e.status == N.NSA_ERR_UNSUPPORTED
        assert math.ceil(max(nsub, 1) / reps_cap) > min(cap, 64)
        return
    CS, CA, gangs = g.scorers_per_row, g.attenders_per_row, g.rows_at_once
    assert g.workgroups == gangs * (CS + CA) <= cap
    assert 1 <= gangs <= rows
    assert 1 <= CS and CS + CA <= 64
    assert CS * g.reps_per_scorer >= nsub and g.reps_per_scorer <= reps_cap
    assert g.reps_per_scorer % 4 == 0          # whole blocks per scorer
    assert CA == 0 or (k_e > 0 and CA <= k_e + 1)
    # block index -> (role, gang, member), as the kernel maps it
    seen = set()
    for b in range(g.workgroups):
        if b < gangs * CS:
            key = ("scorer", b // CS, b % CS)
        else:
            bb = b - gangs * CS
            key = ("attender", bb // CA, bb % CA)
        assert key[1] < gangs
        seen.add(key)
    assert len(seen) == g.workgroups


def test_plan_of_the_long_context_workload():
    """Batch 4 x 8 KV heads at 128K context on 512 resident workgroups: 32
    gangs of 8 scorers (1024 representatives each) and 8 attenders."""
    g = grid_for(4, 32, 8, 128, N.NSA_BF16, 64, 48, 131073, 512)
    assert (g.workgroups, g.scorers_per_row, g.attenders_per_row, g.rows_at_once,
            g.reps_per_scorer) == (512, 8, 8, 32, 1024)


def test_plan_rejects_bad_capacity():
    with pytest.raises(N.NsaError):
        grid_for(4, 32, 8, 128, N.NSA_BF16, 64, 48, 131073, 0)
