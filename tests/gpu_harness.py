"""Shared pieces of the GPU parity tests: upload seeded inputs, drive decode
steps through the C ABI, and compare with the CPU oracle row by row.

Acceptance (stated once here, used by every GPU test):
  * representatives and eviction block scores: bit-identical;
  * eviction set: identical (E is bit-identical on both sides and the rule
    is deterministic on its bits);
  * query-aware blocks: identical except where two competing blocks' oracle
    scores differ by at most 1e-5 relative (near tie), both ways;
  * ordered lists: same set under the same near-tie rule, best first;
  * early-stop position n*: equal, or off by one when the oracle's deciding
    ratio M/A is within 1e-5 relative of tau;
  * outputs: max-abs error against the oracle evaluated on the GPU's blocks,
    2e-2 for bf16 inputs and 1e-4 for float32 inputs.
After every step the oracle takes over the GPU's eviction state, so that one
legal near-tie swap cannot cascade into later steps.
"""

from __future__ import annotations

import math
import os
import sys
from dataclasses import dataclass

import numpy as np
import torch

import workloads as W
from oracle import nsa_oracle as O

NEAR_TIE = 1e-5
TOL = {"bf16": 2e-2, "f32": 1e-4}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def lib():
    import block_sparse_kv_nsa_amd as N
    return N


# ----------------------------------------------------------------------------
# host <-> device
# ----------------------------------------------------------------------------
def to_dev(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def make_layer(cfg: W.Config, batch: W.Batch | None = None, device="cuda"):
    N = lib()
    layer = N.SparseDecodeLayer(
        batch=cfg.batch, num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
        head_dim=cfg.head_dim, max_blocks_per_seq=cfg.max_blocks,
        num_phys_blocks=cfg.num_phys_blocks, dtype=cfg.dtype, mode=cfg.mode, k=cfg.k,
        k_e=cfg.k_e, ordered=cfg.ordered, tau=cfg.tau, device=device)
    if batch is not None:
        upload(layer, cfg, batch)
    return layer


def upload(layer, cfg: W.Config, batch: W.Batch) -> None:
    layer.k_pool.copy_(to_dev(batch.k_pool, cfg.dtype))
    layer.v_pool.copy_(to_dev(batch.v_pool, cfg.dtype))
    layer.block_table.copy_(torch.from_numpy(batch.table))
    layer.evict_logits.copy_(torch.from_numpy(batch.logits))


def device_query(cfg: W.Config, step: int) -> torch.Tensor:
    if cfg.mode.startswith("forecast"):
        return to_dev(W.forecasts(cfg), cfg.dtype)
    return to_dev(W.queries(cfg, step), cfg.dtype)


def device_q(cfg: W.Config, step: int) -> torch.Tensor:
    return to_dev(W.queries(cfg, step), cfg.dtype)


def prefill(layer, cfg: W.Config) -> None:
    dev = layer.device
    nb0 = cfg.nb0
    first = torch.zeros(cfg.batch, dtype=torch.int32, device=dev)
    num = torch.full((cfg.batch,), nb0, dtype=torch.int32, device=dev)
    layer.update_reps(first, num, nb0)


def run_step(layer, cfg: W.Config, step: int, seq_lens=None, fused: bool = False,
             max_seq_len: int | None = None) -> None:
    """One decode step: (the token is already in the pool) reps of a block
    that just filled, then select and decode (two calls, or the fused one).
    max_seq_len: the bound passed to the fused call (default: the longest
    sequence of the step)."""
    dev = layer.device
    L = cfg.seq_len(step)
    lens = np.full(cfg.batch, L, dtype=np.int32) if seq_lens is None else seq_lens
    layer.seq_lens.copy_(torch.from_numpy(lens))
    filled = (lens % 64) == 0
    if filled.any():
        first = torch.from_numpy((lens // 64 - 1).astype(np.int32)).to(dev)
        num = torch.from_numpy(filled.astype(np.int32)).to(dev)
        layer.update_reps(first, num, 1)
    if fused:
        bound = int(lens.max()) if max_seq_len is None else max_seq_len
        layer.step(device_query(cfg, step), device_q(cfg, step), bound)
        return
    layer.select(device_query(cfg, step), int(lens.max()))
    layer.decode(device_q(cfg, step))


def step_error_word(layer) -> int:
    """The fused step's sticky error word (workspace word 2), read raw."""
    torch.cuda.synchronize()
    return int(layer.step_ws[8:12].view(torch.int32).item())


def check_step_status(layer) -> None:
    """Every wait of the fused steps so far ended normally, as the library's
    status query reports it (raises NsaError otherwise)."""
    layer.check_step()
    assert step_error_word(layer) == 0


def step_slot_words(layer, cfg: W.Config) -> torch.Tensor:
    """The fused step's hand-off slots (member statistics, partial (m, l) and
    row keys) as 32-bit words: all zero between calls.  The layout is the
    library's: [256-byte control | stats | (m, l) | acc | keys], member slots
    for 64 members per row, each region 256-byte aligned."""
    def up(x):
        return (x + 255) // 256 * 256
    members = cfg.rows * 64
    off_ml = up(256 + members * cfg.group * 8)
    off_acc = up(off_ml + members * cfg.group * 8)
    off_keys = up(off_acc + members * cfg.group * cfg.head_dim * 4)
    ws = layer.step_ws[:layer.step_ws_bytes]
    return torch.cat([ws[256:off_acc], ws[off_keys:]]).view(torch.int32)


@dataclass
class StepResult:
    selected: np.ndarray
    num_selected: np.ndarray
    evict_set: np.ndarray
    num_processed: np.ndarray
    out: np.ndarray


def fetch(layer) -> StepResult:
    torch.cuda.synchronize()
    return StepResult(layer.selected.cpu().numpy(), layer.num_selected.cpu().numpy(),
                      layer.evict_set.cpu().numpy(), layer.num_processed.cpu().numpy(),
                      to_f64(layer.out))


# ----------------------------------------------------------------------------
# oracle side
# ----------------------------------------------------------------------------
def oracle_row(cfg: W.Config, b: int, g: int, ri: W.RowInputs | None = None) -> O.OracleRow:
    ri = ri or W.row_inputs(cfg, b, g)
    return O.OracleRow(W.stored_to_f64(ri.keys, cfg.dtype), W.stored_to_f64(ri.values, cfg.dtype),
                       ri.logits.astype(np.float64), cfg.dtype, 1.0 / math.sqrt(cfg.head_dim),
                       mode=cfg.mode, k=cfg.k, k_e=cfg.k_e, ordered=cfg.ordered, tau=cfg.tau)


def near(a: float, b: float) -> bool:
    return abs(a - b) <= NEAR_TIE * max(abs(a), abs(b))


def accept_sets(gpu: list, ora: list, score: np.ndarray, what: str) -> None:
    assert len(gpu) == len(ora), f"{what}: |gpu|={len(gpu)} != |oracle|={len(ora)}"
    extra, missing = set(gpu) - set(ora), set(ora) - set(gpu)
    for a in extra:
        for b in missing:
            assert near(score[a], score[b]), (
                f"{what}: gpu picked {a} (S={score[a]!r}) over {b} (S={score[b]!r})")


def check_reps(layer, orow: O.OracleRow, cfg: W.Config, b: int, g: int, nb: int) -> None:
    got = to_f64(layer.reps[b, g, :nb])
    want = orow.reps(nb)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"reps differ at {bad[:5].tolist()} (row {b},{g})"
    if cfg.k_e > 0:
        gE = layer.evict_scores[b, g, :nb].cpu().numpy().astype(np.float64)
        wE = orow.eviction_scores(nb)
        assert np.array_equal(gE, wE), f"E differs (row {b},{g})"


def check_step(cfg: W.Config, res: StepResult, orow: O.OracleRow, b: int, g: int, step: int,
               seq_len: int | None = None, prev: dict | None = None) -> dict:
    """Compare one row of one step; returns bookkeeping for the next step."""
    L = seq_len if seq_len is not None else cfg.seq_len(step)
    nb = L // 64
    G = cfg.group
    q = W.stored_to_f64(W.query_row(cfg, b, g, step), cfg.dtype)
    f = W.stored_to_f64(W.forecast_row(cfg, b, g), cfg.dtype) if cfg.mode.startswith("forecast") else None
    S = orow.scores(nb, q=q, f=f)
    n = int(res.num_selected[b, g])
    gsel = [int(x) for x in res.selected[b, g, :n]]
    assert all(x == -1 for x in res.selected[b, g, n:]), "unused entries must be -1"
    gout = res.out[b, g * G:(g + 1) * G]
    tol = TOL[cfg.dtype]
    info = {"selected": gsel, "tail": nb if L % 64 else None}

    if cfg.ordered:
        ora = O.select_ordered(S, nb, cfg.k).tolist()
        accept_sets(gsel, ora, S, f"ordered list row ({b},{g}) step {step}")
        for i in range(len(gsel) - 1):
            a, c = gsel[i], gsel[i + 1]
            assert S[a] > S[c] or near(S[a], S[c]) or (S[a] == S[c] and a < c), (
                f"ordered list out of order at {i}: {a} ({S[a]!r}) before {c} ({S[c]!r})")
        n_gpu = int(res.num_processed[b, g])
        n_ora, _ = O.early_stop_attention(q, orow.keys, orow.values, gsel, L, cfg.tau, orow.scale)
        if n_gpu != n_ora:
            assert abs(n_gpu - n_ora) == 1 and stop_ratio_near_tau(q, orow, gsel, L, cfg.tau,
                                                                    min(n_gpu, n_ora)), (
                f"n* gpu {n_gpu} oracle {n_ora} row ({b},{g})")
        want = O.sparse_attention(q, orow.keys, orow.values, gsel[:n_gpu], L, orow.scale)
        err = np.abs(gout - want).max()
        assert err <= tol, f"early-stop output err {err} > {tol} row ({b},{g})"
        info["n_star"] = n_gpu
        return info

    st = orow.state
    if cfg.k_e > 0:
        E = orow.eviction_scores(nb)
        ora_ev = O.eviction_update(st.evict_set, st.n_seen, nb, E, cfg.k_e)
        gev = [int(x) for x in res.evict_set[b, g, :min(cfg.k_e, nb)]]
        assert gev == ora_ev.tolist(), f"eviction set differs row ({b},{g}) step {step}"
        ev = np.array(gev, dtype=np.int64)
    else:
        ev = np.zeros(0, dtype=np.int64)
    ora_sel = O.select_blocks(S, ev, nb, cfg.k).tolist()
    assert set(ev.tolist()) <= set(gsel), "eviction set must be selected"
    gq = sorted(set(gsel) - set(ev.tolist()))
    oq = sorted(set(ora_sel) - set(ev.tolist()))
    accept_sets(gq, oq, S, f"query-aware row ({b},{g}) step {step}")
    assert gsel == sorted(gsel), "selected ids must be ascending"
    want = O.sparse_attention(q, orow.keys, orow.values, gsel, L, orow.scale)
    err = np.abs(gout - want).max()
    assert err <= tol, f"output err {err} > {tol} row ({b},{g}) step {step}"
    # re-sync the oracle state to the GPU's
    st.evict_set, st.n_seen = ev, nb
    if prev is not None and cfg.k_e > 0:
        gam = O.locality(gsel, prev["selected"], prev["tail"])
        assert gam >= cfg.k_e / cfg.k - 1e-12, f"gamma {gam} < k_e/k row ({b},{g}) step {step}"
        info["gamma"] = gam
    return info


def stop_ratio_near_tau(q, orow, order, L, tau, n) -> bool:
    """Is the oracle's deciding ratio at list position n within 1e-5 of tau?"""
    nb = L // 64
    toks = [np.arange(nb * 64, L)] + [np.arange(b * 64, b * 64 + 64) for b in order]
    every = np.concatenate(toks).astype(np.int64)
    c = ((q @ orow.keys[every].T) * orow.scale).max(axis=1, keepdims=True)

    def mass(t):
        return np.exp((q @ orow.keys[t].T) * orow.scale - c).sum(axis=1) if t.size else 0 * c[:, 0]

    A = mass(toks[0])
    for i in range(1, n + 1):
        M = mass(toks[i])
        A = A + M
    ratio = M / A
    return bool(np.any(np.abs(ratio - tau) <= NEAR_TIE * tau))


def run_and_check(cfg: W.Config, rows=None, check_every: int = 1, batch=None, row_inputs=None,
                  fused: bool = False, max_len=None):
    """Prefill + every decode step of cfg; compare sampled rows each step.
    max_len: step -> max_seq_len of the fused call (default: the step's)."""
    log(f"[case] {cfg.name}: B={cfg.batch} ctx={cfg.context} Hq={cfg.num_q_heads} "
          f"Hkv={cfg.num_kv_heads} D={cfg.head_dim} {cfg.dtype} {cfg.mode} k={cfg.k} "
          f"k_e={cfg.k_e} ordered={cfg.ordered} steps={cfg.steps} fused={fused}")
    batch = batch if batch is not None else W.build_batch(cfg)
    layer = make_layer(cfg, batch)
    prefill(layer, cfg)
    rows = rows if rows is not None else sample_rows(cfg, 1 << 30)
    orows = {r: oracle_row(cfg, *r, ri=(row_inputs or {}).get(r)) for r in rows}
    torch.cuda.synchronize()
    for r, orow in orows.items():
        check_reps(layer, orow, cfg, *r, cfg.nb0)
    prev = {r: None for r in rows}
    stats = {"gamma_min": 1.0, "n_star": []}
    for t in range(cfg.steps):
        run_step(layer, cfg, t, fused=fused, max_seq_len=None if max_len is None else max_len(t))
        if fused:
            check_step_status(layer)
        L = cfg.seq_len(t)
        # steps where a block fills, and the step after, are always checked
        fill_near = L % 64 == 0 or (L - 1) % 64 == 0
        if t % check_every and t != cfg.steps - 1 and not fill_near:
            # still advance the oracle's eviction state from the GPU's, which
            # must be the oracle's own update (it is deterministic on E)
            res = fetch(layer)
            for r, orow in orows.items():
                if cfg.k_e > 0 and not cfg.ordered:
                    nb = L // 64
                    gev = res.evict_set[r[0], r[1], :min(cfg.k_e, nb)].astype(np.int64)
                    want = O.eviction_update(orow.state.evict_set, orow.state.n_seen, nb,
                                             orow.eviction_scores(nb), cfg.k_e)
                    assert gev.tolist() == want.tolist(), f"eviction set row {r} step {t}"
                    orow.state.evict_set = gev
                    orow.state.n_seen = nb
                prev[r] = {"selected": [int(x) for x in res.selected[r][:res.num_selected[r]]],
                           "tail": L // 64 if L % 64 else None}
            continue
        res = fetch(layer)
        for r, orow in orows.items():
            if L % 64 == 0:
                check_reps(layer, orow, cfg, *r, L // 64)
            info = check_step(cfg, res, orow, r[0], r[1], t, prev=prev[r])
            prev[r] = info
            stats["gamma_min"] = min(stats["gamma_min"], info.get("gamma", 1.0))
            if "n_star" in info:
                stats["n_star"].append(info["n_star"])
    return layer, stats



def replicated_batch(cfg: W.Config, sample):
    """Full-size pools where unsampled rows repeat sampled rows' data (rows
    are independent, so the launch is the full one while only the sampled
    rows are drawn and checked)."""
    ris = {r: W.row_inputs(cfg, *r) for r in sample}
    P, Hh, d = cfg.num_phys_blocks, cfg.num_kv_heads, cfg.head_dim
    dt = W.storage_dtype(cfg)
    k_pool = np.zeros((P, Hh, 64, d), dtype=dt)
    v_pool = np.zeros((P, Hh, 64, d), dtype=dt)
    logits = np.zeros((cfg.batch, Hh, cfg.max_blocks * 64), dtype=np.float32)
    table = W.block_table(cfg)
    order = list(sample)
    for b in range(cfg.batch):
        for g in range(Hh):
            src = (b, g) if (b, g) in ris else order[(b * Hh + g) % len(order)]
            W.scatter_row(cfg, table, b, g, ris[src], k_pool, v_pool, logits)
    return W.Batch(cfg, k_pool, v_pool, logits, table, None), ris



def sample_rows(cfg: W.Config, n: int, seed: int = 7) -> list[tuple[int, int]]:
    rows = [(b, g) for b in range(cfg.batch) for g in range(cfg.num_kv_heads)]
    if len(rows) <= n:
        return rows
    rng = np.random.default_rng(seed)
    pick = sorted(rng.choice(len(rows), n, replace=False).tolist())
    keep = {0, len(rows) - 1}
    return sorted({rows[i] for i in pick} | {rows[i] for i in keep})


def gpu_available() -> bool:
    return torch.cuda.is_available() and os.path.exists(
        os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "block_sparse_kv_nsa_amd", "libnsa.so"))
