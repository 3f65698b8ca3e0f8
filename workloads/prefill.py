"""Seeded synthetic prefill workloads for S2O attention (inputs only).

Attention maps of long-context models are striped: a few key tokens draw
attention from most queries (vertical stripes), and the mass of a query is
concentrated on few tokens (S2O technical summary, "Enunciato del Problema"
and "Significato e Affermazioni").  The draw below gives the prefill that
structure, on top of the key geometry of the decode workloads:

* keys      ``N(0, 0.5^2) + 2*mu``   (``mu`` a seeded unit vector per KV head)
* token 0   key ``-3*mu`` exactly (the sink)
* stripes   each token t >= 1 independently with probability ``stripe_rate``:
            key ``N(0, 0.5^2) + stripe_scale * u`` (``u`` a seeded unit
            vector per KV head)
* queries   ``N(0, 1) + query_scale * u`` of the head's KV head
* values    ``N(0, 1)``

Every tensor is drawn per (sequence b, KV head g) or (sequence b, query head
h) from ``numpy.random.default_rng(SeedSequence([1234, cfg_id, tag, ...]))``.
bf16 tensors are the round-to-nearest-even images of float32 draws, carried as
``uint16`` bit patterns.  Keys and values are laid out in the paged pools of
the decode workloads ([P][Hkv][64][d], through a block table).
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from .synth import _rng, _store, _unit, storage_dtype  # noqa: F401  (shared draw helpers)

TAG_PF_MU, TAG_PF_U, TAG_PF_KEYS, TAG_PF_STRIPE, TAG_PF_VALS, TAG_PF_Q, TAG_PF_TABLE = range(21, 28)


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    cfg_id: int
    batch: int
    seq_len: int            # tokens of each prompt (sequence b has seq_len - b*len_step)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    segment: int            # tokens per segment (a multiple of 64)
    tau: float
    dtype: str = "bf16"
    len_step: int = 0       # ragged batches: sequence b is len_step*b tokens shorter
    stripe_rate: float = 0.01
    stripe_scale: float = 16.0
    query_scale: float = 8.0
    permuted_table: bool = True
    block: int = 64

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def length(self, b: int) -> int:
        return self.seq_len - self.len_step * b

    @property
    def max_blocks(self) -> int:
        return -(-self.seq_len // self.block)

    @property
    def num_phys_blocks(self) -> int:
        return self.batch * self.max_blocks

    @property
    def num_segments(self) -> int:
        return -(-self.seq_len // self.segment)

    def replace(self, **kw) -> "PrefillConfig":
        return dataclasses.replace(self, **kw)


PREFILL_CONFIGS = {
    "s2o-tiny": PrefillConfig("s2o-tiny", 40, batch=2, seq_len=64 * 13 + 37, num_q_heads=4,
                              num_kv_heads=2, head_dim=128, segment=128, tau=1e-3, len_step=200,
                              stripe_rate=0.03),
    "s2o-prefill-32k": PrefillConfig("s2o-prefill-32k", 41, batch=1, seq_len=32768,
                                     num_q_heads=32, num_kv_heads=8, head_dim=128,
                                     segment=1024, tau=1e-3),
}


def prefill_config(name: str, **overrides) -> PrefillConfig:
    c = PREFILL_CONFIGS[name]
    return c.replace(**overrides) if overrides else c


def stripe_direction(cfg: PrefillConfig, g: int) -> np.ndarray:
    return _unit(_rng(cfg.cfg_id, TAG_PF_U, g).standard_normal(cfg.head_dim))


def kv_row(cfg: PrefillConfig, b: int, g: int):
    """Stored keys and values of sequence b, KV head g: ([L][d], [L][d])."""
    L, d = cfg.length(b), cfg.head_dim
    z = _rng(cfg.cfg_id, TAG_PF_KEYS, b, g).standard_normal((L, d), dtype=np.float32)
    mu = _unit(_rng(cfg.cfg_id, TAG_PF_MU, g).standard_normal(d))
    keys = z * np.float32(0.5) + np.float32(2.0) * mu
    stripe = _rng(cfg.cfg_id, TAG_PF_STRIPE, b, g).random(L) < cfg.stripe_rate
    stripe[0] = False
    u = stripe_direction(cfg, g)
    keys[stripe] = z[stripe] * np.float32(0.5) + np.float32(cfg.stripe_scale) * u
    keys[0] = np.float32(-3.0) * mu
    vals = _rng(cfg.cfg_id, TAG_PF_VALS, b, g).standard_normal((L, d), dtype=np.float32)
    return _store(keys, cfg.dtype), _store(vals, cfg.dtype)


def q_row(cfg: PrefillConfig, b: int, h: int) -> np.ndarray:
    """Stored queries of sequence b, query head h: [L][d]."""
    L, d = cfg.length(b), cfg.head_dim
    z = _rng(cfg.cfg_id, TAG_PF_Q, b, h).standard_normal((L, d), dtype=np.float32)
    u = stripe_direction(cfg, h // cfg.group)
    return _store(z + np.float32(cfg.query_scale) * u, cfg.dtype)


def prefill_table(cfg: PrefillConfig) -> np.ndarray:
    """int32 [B][max_blocks]: logical block -> physical pool slot."""
    P = cfg.num_phys_blocks
    slots = _rng(cfg.cfg_id, TAG_PF_TABLE).permutation(P) if cfg.permuted_table else np.arange(P)
    return slots.reshape(cfg.batch, cfg.max_blocks).astype(np.int32)


@dataclass
class PrefillBatch:
    cfg: PrefillConfig
    q: np.ndarray          # [B][Hq][seq_len][d] stored dtype (rows past a sequence's length are 0)
    k_pool: np.ndarray     # [P][Hkv][64][d]
    v_pool: np.ndarray     # [P][Hkv][64][d]
    table: np.ndarray      # [B][max_blocks] int32
    seq_lens: np.ndarray   # [B] int32


def build_prefill(cfg: PrefillConfig, threads: int | None = None) -> PrefillBatch:
    """Draw every sequence and lay it out (host memory)."""
    B, Hq, Hkv, d, blk = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block
    dt = storage_dtype(cfg)
    q = np.zeros((B, Hq, cfg.seq_len, d), dtype=dt)
    k_pool = np.zeros((cfg.num_phys_blocks, Hkv, blk, d), dtype=dt)
    v_pool = np.zeros_like(k_pool)
    table = prefill_table(cfg)

    def kv_work(row):
        b, g = divmod(row, Hkv)
        keys, vals = kv_row(cfg, b, g)
        L = keys.shape[0]
        for j in range(0, L, blk):
            n = min(blk, L - j)
            k_pool[table[b, j // blk], g, :n] = keys[j:j + n]
            v_pool[table[b, j // blk], g, :n] = vals[j:j + n]

    def q_work(row):
        b, h = divmod(row, Hq)
        q[b, h, :cfg.length(b)] = q_row(cfg, b, h)

    n = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max(1, n)) as ex:
        list(ex.map(kv_work, range(B * Hkv)))
        list(ex.map(q_work, range(B * Hq)))
    lens = np.array([cfg.length(b) for b in range(B)], dtype=np.int32)
    return PrefillBatch(cfg, q, k_pool, v_pool, table, lens)
