"""Sanity of the seeded input generators (shapes, ids, draws)."""
import numpy as np

import oracle
import workloads as W
from conftest import load_golden


def _check_tables(case):
    ids = []
    for s, L in enumerate(case.context_lens):
        n = oracle.blocks_for(int(L), case.B)
        row = case.block_tables[s]
        assert (row[:n] >= 0).all() and (row[:n] < case.NB).all()
        assert (row[n:] == -1).all()
        ids.extend(row[:n].tolist())
    assert len(ids) == len(set(ids))


def test_seven_b_case_draws_the_lessons_lengths():
    c = W.seven_b_single_layer()
    assert c.context_lens.tolist() == load_golden("seed7_simulation.json")["lengths"]
    assert c.NB == 407 and c.k_pool.shape == (407, 32, 16, 128)
    _check_tables(c)
    assert c.kv_bytes() == 5126 * 32 * 128 * 4


def test_tiny_case_shapes():
    c = W.tiny_worked_example()
    assert c.context_lens.tolist() == [40, 48] and c.NB == 16 and c.MB == 3
    _check_tables(c)


def test_chat_lengths_and_layer_tables():
    L = W.chat_lengths()
    assert len(L) == 128 and L.min() >= 150 and L.max() <= 2500
    assert int(L.sum()) == 169005 and int(L.max()) == 2400
    c = W.chat_layer(5, lengths=L)
    assert c.k_pool is None and c.NB == W.pool_blocks(sum(oracle.blocks_for(x, 16) for x in L))
    _check_tables(c)
    assert not np.array_equal(c.block_tables, W.chat_layer(6, lengths=L).block_tables)


def test_shared_prefix_layout():
    d = W.shared_prefix()
    B = d["B"]
    assert len(d["shared_ids"]) == oracle.blocks_for(500, B) == 32
    assert d["copy_pairs"].shape == (64, 2)
    assert (d["copy_pairs"][:, 0] == d["shared_ids"][-1]).all()
    for s in range(64):
        L = int(d["context_lens"][s])
        n = oracle.blocks_for(L, B)
        row = d["tables"][s]
        assert (row[:31] == d["shared_ids"][:31]).all()
        assert row[31] == d["copy_pairs"][s, 1]
        assert (row[n:] == -1).all() and (row[:n] >= 0).all()
        assert len(d["suffix_k"][s]) == L - 500
    priv = np.concatenate(d["private_ids"])
    assert len(set(priv.tolist())) == len(priv)
    assert not set(priv.tolist()) & set(d["shared_ids"].tolist())


def test_long_context_pool_is_exactly_full():
    c = W.long_context()
    assert c.NB == 2048 and c.B == 32
    _check_tables(c)
    assert sorted(c.block_tables.reshape(-1).tolist()) == list(range(2048))
