"""The host validator accepts every input the workload generators produce (so
the GPU tests feed the kernels valid data) and rejects each kind of planted
caller mistake."""
import numpy as np
import pytest

import oracle
import workloads as W
from host_validate import InvalidInput, copy_pairs, decode_inputs, prefill_inputs, write_batch


def decode_ok(c):
    decode_inputs(c.block_tables, c.context_lens, c.B, c.NB, c.max_context_len)
    write_batch(oracle.decode_slots(c.block_tables, c.context_lens, c.B, c.NB), c.B, c.NB)


def test_decode_workloads_are_valid():
    decode_ok(W.tiny_worked_example())
    decode_ok(W.seven_b_single_layer())
    decode_ok(W.long_context(with_pools=False))
    for layer in (0, 31):
        decode_ok(W.chat_layer(layer))
    for B in (8, 16, 48, 256):
        decode_ok(W.make_case(f"B{B}", 5000 + B, [1, B - 1, B, B + 1, 700], Hq=4, Hkv=2, B=B,
                              with_pools=False))
    decode_ok(W.chat_layer(0, contiguous=True))


def test_shared_prefix_flow_is_valid():
    d = W.shared_prefix()
    decode_inputs(d["tables"], d["context_lens"], d["B"], d["NB"])
    copy_pairs(d["copy_pairs"], d["NB"])
    seq = np.concatenate([np.full(L - d["prefix_len"], s, np.int32)
                          for s, L in enumerate(d["context_lens"])])
    pos = np.concatenate([np.arange(d["prefix_len"], L, dtype=np.int32) for L in d["context_lens"]])
    write_batch(oracle.token_slots(d["tables"], seq, pos, d["B"], d["NB"]), d["B"], d["NB"])


def test_prefill_workloads_are_valid():
    for c in (W.chat_prefill(with_pools=False),
              W.make_prefill_case("ragged", 3000, [1, 15, 16, 17, 33, 64, 65, 130],
                                  [0, 0, 5, 100, 0, 31, 16, 7], Hq=4, Hkv=2, B=16,
                                  with_pools=False)):
        prefill_inputs(c.block_tables, c.context_lens, c.query_start, c.T, c.B, c.NB,
                       c.max_query_len)
    d = W.prefix_prefill()
    prefill_inputs(d["tables"], d["context_lens"], d["query_start"], len(d["prefill_query"]),
                   d["B"], d["NB"], int(d["new_lens"].max()))


@pytest.fixture()
def case():
    return W.make_case("planted", 5100, [1, 17, 40, 64], Hq=4, Hkv=2, B=16, with_pools=False)


def test_table_entry_outside_the_pool_is_caught(case):
    t = case.block_tables.copy()
    t[2, 1] = case.NB
    with pytest.raises(InvalidInput, match="table entry 1"):
        decode_inputs(t, case.context_lens, case.B, case.NB)
    t[2, 1] = -1
    with pytest.raises(InvalidInput, match="outside"):
        decode_inputs(t, case.context_lens, case.B, case.NB)


def test_unused_table_entries_are_not_checked(case):
    t = case.block_tables.copy()
    t[0, 1:] = 10 ** 6            # sequence 0 has one token: entries past its first are free
    decode_inputs(t, case.context_lens, case.B, case.NB)


def test_length_beyond_the_table_is_caught(case):
    lens = case.context_lens.copy()
    lens[1] = case.MB * case.B + 1
    with pytest.raises(InvalidInput, match="sequence 1"):
        decode_inputs(case.block_tables, lens, case.B, case.NB)
    with pytest.raises(InvalidInput, match="max_context_len"):
        decode_inputs(case.block_tables, case.context_lens, case.B, case.NB, max_context_len=63)


def test_block_twice_in_one_table_is_caught(case):
    t = case.block_tables.copy()
    t[3, 2] = t[3, 0]
    with pytest.raises(InvalidInput, match="twice"):
        decode_inputs(t, case.context_lens, case.B, case.NB)


def test_slot_conflicts_are_caught(case):
    with pytest.raises(InvalidInput, match="same slot"):
        write_batch(np.array([5, -1, 7, 5]), case.B, case.NB)
    with pytest.raises(InvalidInput, match="outside"):
        write_batch(np.array([case.NB * case.B]), case.B, case.NB)
    write_batch(np.array([-1, -1, 3]), case.B, case.NB)   # skips may repeat


def test_copy_pair_conflicts_are_caught():
    copy_pairs(np.array([[3, 4], [3, 5]]), 8)             # one source, two copies: fine
    with pytest.raises(InvalidInput, match="written twice"):
        copy_pairs(np.array([[1, 4], [2, 4]]), 8)
    with pytest.raises(InvalidInput, match="both copied"):
        copy_pairs(np.array([[1, 2], [2, 3]]), 8)
    with pytest.raises(InvalidInput, match="destination"):
        copy_pairs(np.array([[1, 8]]), 8)
    copy_pairs(np.array([[1, 2], [2, 1]]), 8, 8, same_pool=False)   # swap between two pools


def test_prefill_query_ranges_are_checked(case):
    lens = case.context_lens
    qs = np.array([0, 1, 10, 20, 30], np.int32)
    prefill_inputs(case.block_tables, lens, qs, 30, case.B, case.NB, 10)
    with pytest.raises(InvalidInput, match="decreases"):
        prefill_inputs(case.block_tables, lens, np.array([0, 5, 3, 20, 30]), 30, case.B, case.NB, 30)
    with pytest.raises(InvalidInput, match="only L = 1"):
        prefill_inputs(case.block_tables, lens, np.array([0, 2, 10, 20, 30]), 30, case.B, case.NB, 10)
    with pytest.raises(InvalidInput, match="max_query_len"):
        prefill_inputs(case.block_tables, lens, qs, 30, case.B, case.NB, 9)
    with pytest.raises(InvalidInput, match="outside"):
        prefill_inputs(case.block_tables, lens, qs, 29, case.B, case.NB, 10)
