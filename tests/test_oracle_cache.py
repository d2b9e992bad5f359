"""Pins for the oracle's cache writes, block copies and gather."""
import numpy as np
import pytest

import oracle
from conftest import load_golden


def test_write_kv_tiny_hand_example():
    g = load_golden("write_kv_tiny.json")
    NB, H, B, D = g["NB"], g["Hkv"], g["B"], g["D"]
    pool = np.zeros((NB, H, B, D), dtype=np.float32)
    n = len(g["slot_mapping"])
    key = np.array([[[100 * (i + 1) + 10 * h + d for d in range(D)] for h in range(H)]
                    for i in range(n)], dtype=np.float32)
    k, v = oracle.write_kv(pool, pool.copy(), key, key + 0.5, g["slot_mapping"])
    assert k.reshape(-1).tolist() == g["expected_flat_pool"]
    expected_v = np.array(g["expected_flat_pool"], dtype=np.float32)
    expected_v[expected_v != 0] += 0.5
    assert v.reshape(-1).tolist() == expected_v.tolist()
    assert pool.sum() == 0  # input untouched


def test_copy_blocks_tiny_hand_example():
    g = load_golden("copy_tiny.json")
    pool = np.array(g["pool_blocks"], dtype=np.float32).reshape(g["NB"], g["Hkv"], g["B"], g["D"])
    k, v = oracle.copy_blocks(pool, -pool, g["pairs"])
    exp = np.array(g["expected_blocks"], dtype=np.float32).reshape(pool.shape)
    assert np.array_equal(k, exp)
    assert np.array_equal(v, -exp)


def test_copy_reads_sources_before_any_write_and_rejects_bad_pairs():
    pool = np.arange(5, dtype=np.float32).reshape(5, 1, 1, 1)
    with pytest.raises(ValueError):
        oracle.copy_blocks(pool, pool, [[0, 1], [1, 2]])   # 1 is a source and a destination
    with pytest.raises(ValueError):
        oracle.copy_blocks(pool, pool, [[0, 3], [1, 3]])   # duplicate destination
    k, _ = oracle.copy_blocks(pool, pool, [[0, 9], [4, 1]])  # out-of-pool pair skipped
    assert k.reshape(-1).tolist() == [0, 4, 2, 3, 4]


def test_write_skips_negative_and_out_of_pool_slots_and_rejects_duplicates():
    pool = np.zeros((2, 1, 2, 1), dtype=np.float32)
    key = np.array([[[1.0]], [[2.0]], [[3.0]]])
    k, _ = oracle.write_kv(pool, pool, key, key, [-1, 4, 3])
    assert k.reshape(-1).tolist() == [0, 0, 0, 3]
    with pytest.raises(ValueError):
        oracle.write_kv(pool, pool, key, key, [1, 1, 0])


def test_write_then_gather_round_trip_through_a_shuffled_table():
    rng = np.random.default_rng(3)
    NB, H, B, D, L = 12, 3, 4, 8, 27
    nb = oracle.blocks_for(L, B)
    table = rng.permutation(NB)[:nb].astype(np.int32)
    pool = rng.standard_normal((NB, H, B, D)).astype(np.float16)
    keys = rng.standard_normal((L, H, D)).astype(np.float16)
    slots = oracle.token_slots(table[None, :], np.zeros(L, int), np.arange(L), B, NB)
    assert len(set(slots.tolist())) == L
    k, _ = oracle.write_kv(pool, pool, keys, keys, slots)
    seq = oracle.gather(k, table, L, B)            # [H, L, D]
    assert np.array_equal(seq, keys.transpose(1, 0, 2))
    # blocks the table does not name are untouched
    others = np.setdiff1d(np.arange(NB), table)
    assert np.array_equal(k[others], pool[others])


def test_identity_table_with_block_equal_to_length_is_plain_assignment():
    rng = np.random.default_rng(4)
    H, D, L = 2, 4, 6
    pool = np.zeros((1, H, L, D))
    keys = rng.standard_normal((L, H, D))
    k, _ = oracle.write_kv(pool, pool, keys, keys, np.arange(L))
    for t in range(L):
        assert np.array_equal(k[0, :, t, :], keys[t])


def test_gather_rejects_bad_tables():
    pool = np.zeros((4, 1, 2, 1))
    with pytest.raises(ValueError):
        oracle.gather(pool, [0, 7], 3, 2)
    with pytest.raises(ValueError):
        oracle.gather(pool, [0], 3, 2)


def test_swap_blocks_tiny_hand_example():
    g = load_golden("swap_tiny.json")
    shape = lambda blocks: np.array(blocks, dtype=np.float32).reshape(len(blocks), g["Hkv"], g["B"], g["D"])
    src, dst = shape(g["src_blocks"]), shape(g["dst_blocks"])
    k, v = oracle.swap_blocks(dst, dst + 9, src, src * 10, g["pairs"])
    exp = shape(g["expected_dst_blocks"])
    assert np.array_equal(k, exp)
    assert np.array_equal(v[[0, 3]], exp[[0, 3]] * 10) and np.array_equal(v[[1, 2]], dst[[1, 2]] + 9)


def test_swap_out_and_back_in_restores_what_decode_reads():
    rng = np.random.default_rng(12)
    NB, H, B, D, L = 10, 2, 4, 8, 15
    dev_k = rng.standard_normal((NB, H, B, D)).astype(np.float16)
    dev_v = rng.standard_normal((NB, H, B, D)).astype(np.float16)
    table = np.array([7, 1, 4, 9])
    host_k = np.zeros((6, H, B, D), np.float16)
    host_v = np.zeros_like(host_k)
    out_pairs = [[b, i] for i, b in enumerate(table)]            # evict to host slots 0..3
    host_k, host_v = oracle.swap_blocks(host_k, host_v, dev_k, dev_v, out_pairs)
    fresh_k = np.full_like(dev_k, np.nan)
    fresh_v = np.full_like(dev_v, np.nan)
    new_ids = np.array([2, 5, 0, 8])                              # resume into other blocks
    in_pairs = [[i, b] for i, b in enumerate(new_ids)]
    fresh_k, fresh_v = oracle.swap_blocks(fresh_k, fresh_v, host_k, host_v, in_pairs)
    assert np.array_equal(oracle.gather(fresh_k, new_ids, L, B), oracle.gather(dev_k, table, L, B))
    assert np.array_equal(oracle.gather(fresh_v, new_ids, L, B), oracle.gather(dev_v, table, L, B))


def test_swap_within_one_pool_is_copy_on_write():
    rng = np.random.default_rng(13)
    pool = rng.standard_normal((6, 2, 4, 8))
    pairs = [[1, 4], [2, 0]]
    a = oracle.swap_blocks(pool, pool * 2, pool, pool * 2, pairs)
    b = oracle.copy_blocks(pool, pool * 2, pairs)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    with pytest.raises(ValueError):
        oracle.swap_blocks(pool, pool, pool, pool, [[0, 3], [1, 3]])
