"""Seeded synthetic inputs: determinism, per-row independence, layout."""

import numpy as np

import workloads as W


def test_same_seed_same_bytes():
    c = W.config(0)
    a, b = W.row_inputs(c, 0, 0), W.row_inputs(c, 0, 0)
    assert a.keys.tobytes() == b.keys.tobytes()
    assert a.values.tobytes() == b.values.tobytes()
    assert a.logits.tobytes() == b.logits.tobytes()


def test_rows_regenerate_independently():
    c = W.config(1, context=1024, steps=3)
    batch = W.build_batch(c, threads=4)
    for b, g in ((0, 0), (5, 1), (7, 1)):
        ri = W.row_inputs(c, b, g)
        slots = batch.table[b, : c.total_tokens // 64]
        got = batch.k_pool[slots, g].reshape(-1, c.head_dim)
        assert np.array_equal(got, ri.keys[: got.shape[0]])
        assert np.array_equal(batch.logits[b, g, : c.total_tokens], ri.logits)


def test_sink_and_planted_structure():
    c = W.config(0)
    ri = W.row_inputs(c, 0, 0)
    mu = W.key_centre(c, 0)
    assert np.array_equal(ri.keys[0], (np.float32(-3.0) * mu).astype(np.float32))
    assert len(set(ri.planted.tolist())) == 4 and ri.planted.min() >= 1
    assert ri.planted.max() < c.nb0


def test_permuted_table_is_a_permutation():
    c = W.config(3, batch=2, context=64 * 40, steps=3)
    t = W.block_table(c)
    assert sorted(t.ravel().tolist()) == list(range(c.num_phys_blocks))
    assert not np.array_equal(t.ravel(), np.arange(c.num_phys_blocks))


def test_bf16_storage_roundtrip():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3], dtype=np.float32)
    bits = W.f32_to_bf16_bits(x)
    back = W.bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.015625)
    assert back[3] == -2.5
