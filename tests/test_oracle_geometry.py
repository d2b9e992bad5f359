"""Pins for the oracle's block geometry against values the pages print.

Each fixture under tests/golden names the page and section it comes from.
"""
import math

import numpy as np
import pytest

import oracle
from conftest import load_golden


def test_seed7_simulation_matches_printed_output():
    g = load_golden("seed7_simulation.json")
    rng = np.random.default_rng(g["recipe"]["seed"])
    lengths = rng.integers(50, 900, size=g["recipe"]["n_requests"])
    assert lengths.tolist() == g["lengths"]
    B, max_len = g["recipe"]["block"], g["recipe"]["max_len"]
    assert max_len * len(lengths) == g["reserved_slots"]
    assert int(lengths.sum()) == g["used_slots"]
    assert round(100 * oracle.contiguous_waste(lengths, max_len), 1) == g["contiguous_waste_pct_1dp"]
    assert sum(oracle.blocks_for(L, B) for L in lengths) * B == g["paged_allocated_slots"]
    assert round(100 * oracle.paged_waste(lengths, B), 1) == g["paged_waste_pct_1dp"]
    n0 = oracle.blocks_for(lengths[0], B)
    assert n0 == g["request0_blocks"]
    # the printed table is the request's n0 blocks taken one at a time from
    # the end of a shuffled list of 400 ids, after the lengths were drawn
    shuffled = rng.permutation(400)
    table = [int(b) for b in shuffled[::-1][:n0]]
    assert table[:6] == g["request0_table_head"]
    t = g["token"]
    assert oracle.logical_block(t, B) == g["token_logical_block"]
    assert oracle.block_offset(t, B) == g["token_offset"]
    assert table[oracle.logical_block(t, B)] == g["token_physical_block"]
    assert oracle.slot_of(table, t, B) == g["token_physical_block"] * B + g["token_offset"]


def test_lifecycle_walk():
    g = load_golden("lifecycle.json")
    B = g["block"]
    assert oracle.blocks_for(g["prompt_tokens"], B) == g["prompt_blocks"]
    assert oracle.empty_slots(g["prompt_tokens"], B) == g["last_block_empty_slots"]
    t0, t1 = g["last_block_tokens"]
    table = g["table_after_prefill"]
    for t in range(t0, t1 + 1):
        assert table[oracle.logical_block(t, B)] == table[-1]
    # position 48 is past the three blocks: a fourth is needed
    assert oracle.logical_block(48, B) == len(table)
    assert oracle.blocks_for(49, B) == len(g["table_walk"])
    walk = np.array([g["table_walk"]], dtype=np.int32)
    pos = np.arange(40, 49)
    slots = oracle.token_slots(walk, np.zeros(9, int), pos, B, NB=16)
    assert slots.tolist() == g["derived_slots_positions_40_to_48"]
    assert slots[-1] // B == g["new_block_for_token_48"]


def test_block_size_tradeoff():
    g = load_golden("block_size_tradeoff.json")
    L = g["tokens"]
    for B, nb, empty in zip(g["block_sizes"], g["blocks"], g["empty_slots"]):
        assert oracle.blocks_for(L, B) == nb
        assert oracle.empty_slots(L, B) == empty
    assert round(100 * 168 / (3 * 256)) == g["waste_pct_at_256_rounded"]
    per_tok = oracle.kv_bytes_per_token(32, 32, 128, 2)
    assert per_tok == g["kib_per_token"] * 1024
    assert oracle.empty_slots(L, 16) * per_tok == g["waste_mib_at_16"] * 2**20
    assert oracle.empty_slots(L, 256) * per_tok == g["waste_mib_at_256"] * 2**20


def test_chat_sizing():
    g = load_golden("sizing.json")
    e = g["kv_entry"]
    assert oracle.kv_bytes_per_token(e["layers"], e["kv_heads"], e["head_dim"],
                                     e["elem_bytes"]) == e["kib_per_token"] * 1024
    c = g["chat"]
    B = c["block"]
    assert oracle.blocks_for(c["avg_prompt_tokens"], B) == c["avg_prompt_blocks"]
    assert oracle.blocks_for(c["avg_generation_tokens"], B) == c["avg_generation_blocks"]
    assert c["avg_prompt_blocks"] + c["avg_generation_blocks"] == c["blocks_per_request"]
    assert c["users"] * c["blocks_per_request"] == c["peak_blocks"]
    assert oracle.blocks_for(c["shared_prompt_tokens"], B) == c["shared_prompt_blocks"]
    sc = load_golden("pause_and_think.json")["support_chatbot"]
    assert oracle.blocks_for(sc["system_prompt_tokens"], sc["block"]) == sc["blocks"]


def test_blocks_for_is_the_integer_ceiling():
    # brute force against the float ceiling, exact for these small integers
    for B in (1, 2, 3, 16, 32, 64):
        for L in range(0, 300):
            n = oracle.blocks_for(L, B)
            assert n == math.ceil(L / B)
            assert n * B >= L and (n - 1) * B < L or L == 0
    with pytest.raises(ValueError):
        oracle.blocks_for(5, 0)


def test_slot_translation_visits_every_slot_of_the_table_once():
    # a sequence filling its blocks exactly covers each table block's slots once
    rng = np.random.default_rng(0)
    B, NB = 4, 10
    table = rng.permutation(NB)[:5]
    slots = [oracle.slot_of(table, t, B) for t in range(5 * B)]
    expected = sorted(int(b) * B + o for b in table for o in range(B))
    assert sorted(slots) == expected
    # consecutive tokens inside a block sit in consecutive slots
    for t in range(5 * B - 1):
        if (t + 1) % B:
            assert slots[t + 1] == slots[t] + 1


def test_decode_slots_and_invalid_inputs():
    tables = np.array([[3, 1, -1], [0, 2, 5], [7, -1, -1]], dtype=np.int32)
    lens = np.array([5, 12, 0])
    got = oracle.decode_slots(tables, lens, B=4, NB=6)
    # seq 0: position 4 -> logical block 1 -> block 1 -> slot 4; seq 1: position 11 -> block 5,
    # offset 3 -> 23; seq 2: empty
    assert got.tolist() == [4, 23, -1]
    # entry outside the pool and position past the row both give -1
    assert oracle.decode_slots(tables, [1], B=4, NB=3).tolist() == [-1]
    assert oracle.decode_slots(tables, [13], B=4, NB=8).tolist() == [-1]
    assert oracle.token_slots(tables, [1, 9], [11, 0], B=4, NB=6).tolist() == [23, -1]
