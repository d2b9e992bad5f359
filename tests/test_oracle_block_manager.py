"""Pins for the host block-manager fixture (reference counts, copy-on-write)
against the lesson's printed practice trace and its pause-and-think answers."""
import pytest

import oracle
from conftest import load_golden


def _refs(m):
    return {str(b): c for b, c in enumerate(m.count) if c > 0}


def _filled(m, n):
    s = m.new_sequence()
    for _ in range(n):
        m.append(s)
    return s


def test_practice_trace_matches_printed_output():
    g = load_golden("practice_trace.json")
    m = oracle.BlockManager(g["pool_blocks"], g["block"])
    a = _filled(m, g["prompt_tokens"])
    b = m.fork(a)
    assert (a.blocks, b.blocks, _refs(m)) == (g["after_fork"]["A"], g["after_fork"]["B"],
                                              g["after_fork"]["refs"])
    m.append(a)
    s = g["after_A_writes"]
    assert (a.blocks, b.blocks, _refs(m)) == (s["A"], s["B"], s["refs"])
    m.append(b)
    s = g["after_B_writes"]
    assert (a.blocks, b.blocks, _refs(m)) == (s["A"], s["B"], s["refs"])
    assert m.blocks_in_use() == g["blocks_in_use"] < g["blocks_with_two_full_copies"]
    assert m.copies == [(1, 2)]      # only A's write copied


def test_four_samples_share_a_partial_block():
    g = load_golden("pause_and_think.json")["four_samples"]
    B = g["block"]
    m = oracle.BlockManager(16, B)
    a = _filled(m, B + g["last_block_tokens"])
    others = [m.fork(a) for _ in range(g["samples"] - 1)]
    last = a.blocks[-1]
    assert m.refcount(last) == g["samples"]
    slot = m.append(a)
    assert m.copies == [(last, a.blocks[-1])] and a.blocks[-1] != last
    assert slot % B == g["slot_written_in_copy"]
    assert m.refcount(last) == g["original_refs_after"]
    assert all(o.blocks[-1] == last for o in others)     # the full earlier block stays shared
    assert m.refcount(a.blocks[0]) == g["samples"]


def test_second_writer_after_copy_writes_in_place():
    g = load_golden("pause_and_think.json")["second_writer_after_copy"]
    m = oracle.BlockManager(8, 4)
    a = _filled(m, 6)
    b = m.fork(a)
    m.append(a)
    n_copies = len(m.copies)
    assert m.refcount(b.blocks[-1]) == g["reason_refcount"]
    slot = m.append(b)
    assert (len(m.copies) > n_copies) == g["copies"]
    assert slot == b.blocks[-1] * 4 + 2


def test_fifty_chats_one_ends_frees_nothing_shared():
    g = load_golden("pause_and_think.json")["fifty_chats"]
    sc = load_golden("pause_and_think.json")["support_chatbot"]
    m = oracle.BlockManager(400, sc["block"])
    prompt = _filled(m, sc["system_prompt_tokens"])
    assert len(prompt.blocks) == g["shared_blocks"] == sc["blocks"]
    chats = [m.fork(prompt) for _ in range(g["chats"])]
    m.free(prompt)                # the prompt's owner steps away; 50 chats remain
    for c in chats:
        m.append(c)               # each chat's first reply token takes a block of its own
    shared = set(chats[1].blocks[:g["shared_blocks"]])
    freed = m.free(chats[0])
    assert len([b for b in freed if b in shared]) == g["blocks_freed_when_one_ends"]
    assert all(m.refcount(b) == g["refs_after"] for b in shared)
    assert len(freed) == 1        # only the chat's private block returns


def test_full_last_block_takes_a_fresh_block_without_copy():
    m = oracle.BlockManager(8, 4)
    a = _filled(m, 8)
    m.fork(a)
    m.append(a)
    assert m.copies == [] and a.blocks == [0, 1, 2] and a.length == 9


def test_release_returns_blocks_and_exhaustion_changes_nothing():
    m = oracle.BlockManager(3, 2)
    a = _filled(m, 6)
    with pytest.raises(oracle.PoolExhausted):
        m.append(a)
    assert a.blocks == [0, 1, 2] and a.length == 6
    b = m.fork(a)
    m.free(a)
    with pytest.raises(oracle.PoolExhausted):   # full last block, no free block
        m.append(b)
    assert m.copies == [] and b.length == 6
    assert m.free(b) == [0, 1, 2]
    assert m.blocks_in_use() == 0 and list(m.free_list) == [0, 1, 2]


def test_copy_on_write_exhaustion_changes_nothing():
    m = oracle.BlockManager(2, 4)
    a = _filled(m, 6)                 # blocks 0 and 1, the last one half full
    b = m.fork(a)
    with pytest.raises(oracle.PoolExhausted):
        m.append(a)                   # needs a copy of block 1, none free
    assert a.blocks == b.blocks == [0, 1] and m.refcount(1) == 2 and m.copies == []


def test_slots_follow_positions_through_the_table():
    # token t of a sequence lands at offset t % B of the block its table lists
    # at index t // B ([L], "How PagedAttention works", steps 1-3)
    m = oracle.BlockManager(12, 4)
    a, b = m.new_sequence(), m.new_sequence()
    slots = {"a": [], "b": []}
    for step in range(18):
        slots["a"].append(m.append(a))
        if step % 3 == 0:
            slots["b"].append(m.append(b))
    for name, s in (("a", a), ("b", b)):
        for t, slot in enumerate(slots[name]):
            assert slot == oracle.slot_of(s.blocks, t, 4)
