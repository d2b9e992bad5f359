"""The native host block manager (pa_bm_* in the C ABI) against the lesson's
printed trace, its pause-and-think answers, and the oracle's manager under
random operation sequences (bit-exact: slots, copy pairs, tables, counts and
free-list order). Host only: no GPU needed."""
import numpy as np
import pytest

import oracle
from conftest import load_golden


@pytest.fixture(scope="module")
def pa():
    import paged_kv_cache_151_amd as pa
    return pa


def _refs(m, n):
    return {str(b): m.refcount(b) for b in range(n) if m.refcount(b) > 0}


def test_practice_trace(pa):
    g = load_golden("practice_trace.json")
    m = pa.BlockManager(g["pool_blocks"], g["block"])
    a = m.add_sequence()
    for _ in range(g["prompt_tokens"]):
        m.append_tokens([a])
    b = m.fork(a)
    tab = lambda s: m.table(s)[0].tolist()
    assert (tab(a), tab(b), _refs(m, 8)) == (g["after_fork"]["A"], g["after_fork"]["B"],
                                             g["after_fork"]["refs"])
    _, copies = m.append_tokens([a])
    s = g["after_A_writes"]
    assert (tab(a), tab(b), _refs(m, 8)) == (s["A"], s["B"], s["refs"])
    assert copies.tolist() == [[1, 2]]
    _, copies = m.append_tokens([b])
    s = g["after_B_writes"]
    assert (tab(a), tab(b), _refs(m, 8)) == (s["A"], s["B"], s["refs"])
    assert copies.size == 0
    assert 8 - m.num_free() == g["blocks_in_use"]


def test_four_samples_and_fifty_chats(pa):
    g = load_golden("pause_and_think.json")
    f = g["four_samples"]
    B = f["block"]
    m = pa.BlockManager(16, B)
    a = m.add_sequence()
    m.append_tokens([a] * (B + f["last_block_tokens"]))
    for _ in range(f["samples"] - 1):
        m.fork(a)
    last = int(m.table(a)[0][-1])
    slots, copies = m.append_tokens([a])
    assert copies.tolist() == [[last, int(m.table(a)[0][-1])]]
    assert slots[0] % B == f["slot_written_in_copy"]
    assert m.refcount(last) == f["original_refs_after"]

    c = g["fifty_chats"]
    sc = g["support_chatbot"]
    m = pa.BlockManager(400, sc["block"])
    prompt = m.add_sequence()
    m.append_tokens([prompt] * sc["system_prompt_tokens"])
    shared = m.table(prompt)[0]
    assert len(shared) == c["shared_blocks"]
    chats = [m.fork(prompt) for _ in range(c["chats"])]
    m.release(prompt)
    m.append_tokens(chats)
    freed = m.release(chats[0])
    assert freed == 1                      # only that chat's own block
    assert all(m.refcount(int(b)) == c["refs_after"] for b in shared)


def test_export_matches_tables_and_feeds_decode_layout(pa):
    m = pa.BlockManager(32, 16)
    seqs = [m.add_sequence() for _ in range(3)]
    for s, n in zip(seqs, (40, 1, 33)):
        m.append_tokens([s] * n)
    tables, lens = m.export(seqs, 4)
    assert lens.tolist() == [40, 1, 33]
    for i, s in enumerate(seqs):
        row, nt = m.table(s)
        assert tables[i, :len(row)].tolist() == row.tolist() and (tables[i, len(row):] == -1).all()
        assert nt == lens[i]
    with pytest.raises(pa.PaError, match="PA_ERR_SHAPE"):
        m.export(seqs, 2)


def test_exhaustion_applies_a_prefix_and_bad_ids_are_rejected(pa):
    m = pa.BlockManager(3, 2)
    a, b = m.add_sequence(), m.add_sequence()
    with pytest.raises(pa.PaError, match="PA_ERR_EXHAUSTED") as ei:
        m.append_tokens([a, b, a, b, a, b, a])   # 7 tokens need 4 blocks of 2
    assert ei.value.n_applied == 5 and ei.value.slots.tolist() == [0, 2, 1, 3, 4]
    assert m.table(a)[1] == 3 and m.table(b)[1] == 2
    with pytest.raises(pa.PaError, match="PA_ERR_STATE"):
        m.append_tokens([7])
    m.release(a)
    with pytest.raises(pa.PaError, match="PA_ERR_STATE"):
        m.release(a)
    c = m.add_sequence()
    assert c == a                          # the smallest released id is reused
    capped = pa.BlockManager(10, 2, max_blocks_per_seq=2)
    s = capped.add_sequence()
    capped.append_tokens([s] * 4)
    with pytest.raises(pa.PaError, match="PA_ERR_STATE"):
        capped.append_tokens([s])
    with pytest.raises(ValueError, match="1-D list of ids"):   # would be read as a flat list
        capped.append_tokens([[s, s]])
    with pytest.raises(ValueError, match="1-D list of ids"):
        capped.export([[s]], 4)


def _run_random(pa, seed, n_ops=400, NB=40, B=4):
    rng = np.random.default_rng(seed)
    nat = pa.BlockManager(NB, B)
    ref = oracle.BlockManager(NB, B)
    live = {}            # native id -> oracle sequence
    for _ in range(n_ops):
        op = rng.random()
        if op < 0.15 or not live:
            sid = nat.add_sequence()
            live[sid] = ref.new_sequence()
        elif op < 0.25:
            parent = int(rng.choice(list(live)))
            sid = nat.fork(parent)
            live[sid] = ref.fork(live[parent])
        elif op < 0.35 and len(live) > 1:
            sid = int(rng.choice(list(live)))
            freed = nat.release(sid)
            assert freed == len(ref.free(live.pop(sid)))
        else:
            ids = [int(x) for x in rng.choice(list(live), size=int(rng.integers(1, 6)))]
            copies_before = len(ref.copies)
            want_slots = []
            try:
                for sid in ids:
                    want_slots.append(ref.append(live[sid]))
                exhausted = False
            except oracle.PoolExhausted:
                exhausted = True
            want_copies = ref.copies[copies_before:]
            if exhausted:
                with pytest.raises(pa.PaError, match="PA_ERR_EXHAUSTED") as ei:
                    nat.append_tokens(ids)
                assert ei.value.n_applied == len(want_slots)
                assert ei.value.slots.tolist() == want_slots
                assert [tuple(p) for p in ei.value.copy_pairs.tolist()] == want_copies
            else:
                slots, copies = nat.append_tokens(ids)
                assert slots.tolist() == want_slots
                assert [tuple(p) for p in copies.tolist()] == want_copies
        for sid, seq in live.items():
            row, n_tokens = nat.table(sid)
            assert row.tolist() == seq.blocks and n_tokens == seq.length
        assert nat.num_free() == len(ref.free_list)
        for b in range(NB):
            assert nat.refcount(b) == ref.refcount(b)


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_match_the_oracle_manager(pa, seed):
    _run_random(pa, seed)
