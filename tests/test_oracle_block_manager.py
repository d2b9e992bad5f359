"""Pins for the host block-manager fixture (reference counts, copy-on-write)
against the lesson's printed practice trace and its pause-and-think answers."""
import pytest

import oracle
from conftest import load_golden


def _refs(m):
    return {str(k): v for k, v in sorted(m.refs.items())}


def test_practice_trace_matches_printed_output():
    g = load_golden("practice_trace.json")
    m = oracle.BlockManager(g["pool_blocks"], g["block"])
    a = []
    for _ in range(g["prompt_tokens"]):
        m.append_token(a)
    b = m.fork(a)
    assert (a, b, _refs(m)) == (g["after_fork"]["A"], g["after_fork"]["B"], g["after_fork"]["refs"])
    m.append_token(a)
    s = g["after_A_writes"]
    assert (a, b, _refs(m)) == (s["A"], s["B"], s["refs"])
    m.append_token(b)
    s = g["after_B_writes"]
    assert (a, b, _refs(m)) == (s["A"], s["B"], s["refs"])
    assert m.blocks_in_use() == g["blocks_in_use"] < g["blocks_with_two_full_copies"]
    assert m.copies == [(1, 2)]      # only A's write copied


def test_four_samples_share_a_partial_block():
    g = load_golden("pause_and_think.json")["four_samples"]
    B = g["block"]
    m = oracle.BlockManager(16, B)
    a = []
    for _ in range(B + g["last_block_tokens"]):
        m.append_token(a)
    others = [m.fork(a) for _ in range(g["samples"] - 1)]
    last = a[-1]
    assert m.refs[last] == g["samples"]
    slot = m.append_token(a)
    assert m.copies == [(last, a[-1])] and a[-1] != last
    assert slot % B == g["slot_written_in_copy"]
    assert m.refs[last] == g["original_refs_after"]
    assert all(o[-1] == last for o in others)     # the full earlier block stays shared
    assert m.refs[a[0]] == g["samples"]


def test_second_writer_after_copy_writes_in_place():
    m = oracle.BlockManager(8, 4)
    a = []
    for _ in range(6):
        m.append_token(a)
    b = m.fork(a)
    m.append_token(a)
    n_copies = len(m.copies)
    slot = m.append_token(b)
    assert len(m.copies) == n_copies
    assert slot == b[-1] * 4 + 2


def test_fifty_chats_one_ends_frees_nothing_shared():
    g = load_golden("pause_and_think.json")["fifty_chats"]
    sc = load_golden("pause_and_think.json")["support_chatbot"]
    B = sc["block"]
    m = oracle.BlockManager(400, B)
    prompt = []
    for _ in range(sc["system_prompt_tokens"]):
        m.append_token(prompt)
    assert len(prompt) == g["shared_blocks"]
    chats = [m.fork(prompt) for _ in range(g["chats"])]
    m.release(prompt)             # the prompt's owner steps away; 50 chats remain
    for c in chats:
        m.append_token(c)         # each chat's first reply token takes a block of its own
    freed = m.release(chats[0])
    shared_freed = [b for b in freed if b in chats[1]]
    assert len(shared_freed) == g["blocks_freed_when_one_ends"]
    assert all(m.refs[b] == g["refs_after"] for b in chats[1][:g["shared_blocks"]])
    assert len(freed) == 1        # only the chat's private block returns


def test_full_last_block_takes_a_fresh_block_without_copy():
    m = oracle.BlockManager(8, 4)
    a = []
    for _ in range(8):
        m.append_token(a)
    m.fork(a)
    m.append_token(a)
    assert m.copies == [] and a == [0, 1, 2]


def test_release_returns_blocks_and_exhaustion_raises():
    m = oracle.BlockManager(3, 2)
    a = []
    for _ in range(6):
        m.append_token(a)
    with pytest.raises(oracle.PoolExhausted):
        m.append_token(a)
    assert sorted(m.release(a)) == [0, 1, 2]
    assert m.blocks_in_use() == 0
