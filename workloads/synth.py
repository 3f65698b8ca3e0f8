"""Seeded synthetic decode workloads (inputs only).

Every tensor is drawn per row -- one row is one (sequence b, KV head g) -- from
``numpy.random.default_rng(SeedSequence([1234, cfg_id, tag, b, g, ...]))`` so
that any row can be regenerated on its own without holding the whole context.

Distributions follow the key geometry reported for long-context models in the
MagicPIG article ("TopK Attention 的问题" section: the sink token's states are
input-invariant, the key centre direction is stable, and the key centre points
almost opposite the sink key):

* keys      ``N(0, 0.5^2) + 2*mu``   (``mu`` a seeded unit vector per KV head)
* token 0   key ``-3*mu`` exactly (the sink)
* planted   ``n_planted`` blocks per row (drawn from 1..nb0-1) whose keys are
            ``N(0, 0.5^2) + s*u`` with ``u`` the unit direction of the step-0
            query summed over the row's query heads (or of the forecast vector
            in forecast mode) and ``s = planted_scale`` (2 by default)
* values, queries, forecast vectors, eviction logits: ``N(0, 1)``

bf16 tensors are the round-to-nearest-even bf16 images of float32 draws and
are carried as ``uint16`` bit patterns (numpy has no bfloat16).
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BASE_SEED = 1234
TAG_MU, TAG_KEYS, TAG_VALS, TAG_LOGITS, TAG_PLANT, TAG_Q, TAG_F, TAG_TABLE = range(1, 9)


# ----------------------------------------------------------------------------
# bf16 storage helpers (format conversion of inputs, not method arithmetic)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values (float32, or bf16 bits) exactly to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    return np.ascontiguousarray(x32, dtype=np.float32)


# ----------------------------------------------------------------------------
# Configurations
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    batch: int
    context: int          # tokens already cached before decode step 0
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str            # "f32" or "bf16"
    mode: str             # "group_softmax" (NOSA), "forecast" or "forecast_window" (SparDA)
    k: int                # blocks selected per row (the cap in ordered mode)
    k_e: int              # eviction budget (query-agnostic part)
    steps: int            # decode steps; step t appends token context+t
    ordered: bool = False  # emit blocks by descending score (early-stop mode)
    tau: float = 0.0       # early-stop threshold (ordered mode only)
    permuted_table: bool = False
    planted_scale: float = 2.0
    n_planted: int = 4
    block: int = 64
    sub_block: int = 16

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def rows(self) -> int:
        return self.batch * self.num_kv_heads

    @property
    def total_tokens(self) -> int:
        return self.context + self.steps

    @property
    def max_blocks(self) -> int:
        return -(-self.total_tokens // self.block)

    @property
    def num_phys_blocks(self) -> int:
        return self.batch * self.max_blocks

    @property
    def nb0(self) -> int:
        return self.context // self.block

    def seq_len(self, step: int) -> int:
        """Tokens cached once step ``step`` has appended its token."""
        return self.context + step + 1

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    0: Config("tiny-fp32", 0, batch=1, context=4096, num_q_heads=4, num_kv_heads=1,
              head_dim=64, dtype="f32", mode="group_softmax", k=16, k_e=8, steps=1),
    1: Config("nosa-1b", 1, batch=8, context=16384, num_q_heads=16, num_kv_heads=2,
              head_dim=128, dtype="bf16", mode="group_softmax", k=64, k_e=48, steps=32),
    2: Config("sparda-8b", 2, batch=32, context=32768, num_q_heads=32, num_kv_heads=8,
              head_dim=128, dtype="bf16", mode="forecast", k=32, k_e=0, steps=1),
    3: Config("long-128k", 3, batch=4, context=131072, num_q_heads=32, num_kv_heads=8,
              head_dim=128, dtype="bf16", mode="group_softmax", k=64, k_e=48, steps=16,
              permuted_table=True),
    4: Config("early-stop", 4, batch=64, context=65536, num_q_heads=32, num_kv_heads=8,
              head_dim=128, dtype="bf16", mode="group_softmax", k=256, k_e=0, steps=1,
              ordered=True, tau=1e-3),
}


def config(cfg_id: int, **overrides) -> Config:
    c = CONFIGS[cfg_id]
    return c.replace(**overrides) if overrides else c


# ----------------------------------------------------------------------------
# Per-row draws
# ----------------------------------------------------------------------------
def _rng(*parts: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([BASE_SEED, *[int(p) for p in parts]]))


def _unit(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return (v / np.linalg.norm(v)).astype(np.float32)


def key_centre(cfg: Config, g: int) -> np.ndarray:
    """The seeded unit vector mu of KV head g (shared across the batch)."""
    return _unit(_rng(cfg.cfg_id, TAG_MU, g).standard_normal(cfg.head_dim))


def query_row(cfg: Config, b: int, g: int, step: int) -> np.ndarray:
    """Stored queries of the row's G query heads at decode step ``step``: [G][d]."""
    z = _rng(cfg.cfg_id, TAG_Q, b, g, step).standard_normal((cfg.group, cfg.head_dim),
                                                            dtype=np.float32)
    return _store(z, cfg.dtype)


def forecast_row(cfg: Config, b: int, g: int) -> np.ndarray:
    """Stored forecast vector of the row's KV head: [d]."""
    z = _rng(cfg.cfg_id, TAG_F, b, g).standard_normal(cfg.head_dim, dtype=np.float32)
    return _store(z, cfg.dtype)


def planted_direction(cfg: Config, b: int, g: int) -> np.ndarray:
    if cfg.mode.startswith("forecast"):
        v = stored_to_f64(forecast_row(cfg, b, g), cfg.dtype)
    else:
        v = stored_to_f64(query_row(cfg, b, g, 0), cfg.dtype).sum(axis=0)
    return _unit(v)


@dataclass
class RowInputs:
    keys: np.ndarray      # [total_tokens][d] stored dtype
    values: np.ndarray    # [total_tokens][d] stored dtype
    logits: np.ndarray    # [total_tokens] float32 eviction-head logits
    planted: np.ndarray   # [n_planted] int64 logical block ids


def planted_blocks(cfg: Config, b: int, g: int) -> np.ndarray:
    nb0 = cfg.nb0
    n = min(cfg.n_planted, max(nb0 - 1, 0))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(cfg.cfg_id, TAG_PLANT, b, g).choice(np.arange(1, nb0), n, replace=False))


def row_inputs(cfg: Config, b: int, g: int) -> RowInputs:
    T, d = cfg.total_tokens, cfg.head_dim
    z = _rng(cfg.cfg_id, TAG_KEYS, b, g).standard_normal((T, d), dtype=np.float32)
    mu = key_centre(cfg, g)
    keys = z * np.float32(0.5) + np.float32(2.0) * mu
    planted = planted_blocks(cfg, b, g)
    if planted.size:
        u = planted_direction(cfg, b, g)
        shift = np.float32(cfg.planted_scale) * u
        for blk in planted:
            s = slice(blk * cfg.block, (blk + 1) * cfg.block)
            keys[s] = z[s] * np.float32(0.5) + shift
    keys[0] = np.float32(-3.0) * mu
    vals = _rng(cfg.cfg_id, TAG_VALS, b, g).standard_normal((T, d), dtype=np.float32)
    logits = _rng(cfg.cfg_id, TAG_LOGITS, b, g).standard_normal(T, dtype=np.float32)
    return RowInputs(_store(keys, cfg.dtype), _store(vals, cfg.dtype), logits, planted)


# ----------------------------------------------------------------------------
# Paged layout
# ----------------------------------------------------------------------------
def block_table(cfg: Config) -> np.ndarray:
    """int32 [B][max_blocks]: logical block -> physical pool slot."""
    P = cfg.num_phys_blocks
    if cfg.permuted_table:
        slots = _rng(cfg.cfg_id, TAG_TABLE).permutation(P)
    else:
        slots = np.arange(P)
    return slots.reshape(cfg.batch, cfg.max_blocks).astype(np.int32)


def storage_dtype(cfg: Config):
    return np.uint16 if cfg.dtype == "bf16" else np.float32


@dataclass
class Batch:
    cfg: Config
    k_pool: np.ndarray        # [P][Hkv][64][d] stored dtype
    v_pool: np.ndarray        # [P][Hkv][64][d]
    logits: np.ndarray        # [B][Hkv][max_blocks*64] float32, logical token order
    table: np.ndarray         # [B][max_blocks] int32
    planted: np.ndarray       # [B][Hkv][n_planted] int64


def scatter_row(cfg: Config, table: np.ndarray, b: int, g: int, ri: RowInputs,
                k_pool: np.ndarray, v_pool: np.ndarray, logits: np.ndarray) -> None:
    T, blk, d = cfg.total_tokens, cfg.block, cfg.head_dim
    nfull = T // blk
    slots = table[b, :nfull]
    k_pool[slots, g] = ri.keys[: nfull * blk].reshape(nfull, blk, d)
    v_pool[slots, g] = ri.values[: nfull * blk].reshape(nfull, blk, d)
    rem = T - nfull * blk
    if rem:
        s = table[b, nfull]
        k_pool[s, g, :rem] = ri.keys[nfull * blk:]
        v_pool[s, g, :rem] = ri.values[nfull * blk:]
    logits[b, g, :T] = ri.logits


def build_batch(cfg: Config, threads: int | None = None) -> Batch:
    """Draw every row and lay it out in the paged pools (host memory)."""
    P, H, d = cfg.num_phys_blocks, cfg.num_kv_heads, cfg.head_dim
    dt = storage_dtype(cfg)
    k_pool = np.zeros((P, H, cfg.block, d), dtype=dt)
    v_pool = np.zeros((P, H, cfg.block, d), dtype=dt)
    logits = np.zeros((cfg.batch, H, cfg.max_blocks * cfg.block), dtype=np.float32)
    table = block_table(cfg)
    planted = np.zeros((cfg.batch, H, min(cfg.n_planted, max(cfg.nb0 - 1, 0))), dtype=np.int64)

    def work(row):
        b, g = divmod(row, H)
        ri = row_inputs(cfg, b, g)
        scatter_row(cfg, table, b, g, ri, k_pool, v_pool, logits)
        planted[b, g] = ri.planted

    n = threads or min(16, os.cpu_count() or 1)
    if n <= 1 or cfg.rows == 1:
        for r in range(cfg.rows):
            work(r)
    else:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(work, range(cfg.rows)))
    return Batch(cfg, k_pool, v_pool, logits, table, planted)


def queries(cfg: Config, step: int) -> np.ndarray:
    """Stored queries of every row at ``step``: [B][Hq][d]."""
    out = np.zeros((cfg.batch, cfg.num_q_heads, cfg.head_dim), dtype=storage_dtype(cfg))
    G = cfg.group
    for b in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            out[b, g * G:(g + 1) * G] = query_row(cfg, b, g, step)
    return out


def forecasts(cfg: Config) -> np.ndarray:
    """Stored forecast vectors of every row: [B][Hkv][d]."""
    out = np.zeros((cfg.batch, cfg.num_kv_heads, cfg.head_dim), dtype=storage_dtype(cfg))
    for b in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            out[b, g] = forecast_row(cfg, b, g)
    return out
