"""Parity of pa_prefill (HIP, MFMA) against the fp64 CPU oracle: ragged chunks of
new tokens with and without a cached prefix, every grouped-query size, block
sizes 8/16/32/48, the shared-prefix flow (copy-on-write, suffix writes, prefill),
and the invariants that hold bit for bit on the GPU (relabelling blocks,
poison in unused slots, chunked versus one-pass prefill)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_attention_close, dev, host, pa_module, say, u16
from host_validate import prefill_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return pa_module()


def run(pa, c, k_pool=None, v_pool=None, tables=None, out=None, max_query_len=None):
    kp = dev(c.k_pool if k_pool is None else k_pool)
    vp = dev(c.v_pool if v_pool is None else v_pool)
    t = dev(c.block_tables if tables is None else tables)
    o = pa.pa_prefill(dev(c.query), kp, vp, t, dev(c.context_lens), dev(c.query_start),
                      c.max_query_len if max_query_len is None else max_query_len, c.scale,
                      out=None if out is None else dev(out))
    return host(o)


def ref(c, k_pool=None, v_pool=None, tables=None):
    return oracle.prefill(c.query, c.k_pool if k_pool is None else k_pool,
                          c.v_pool if v_pool is None else v_pool,
                          c.block_tables if tables is None else tables, c.context_lens,
                          c.query_start, c.scale)


def check(pa, c):
    say(c.name, f"S={c.S} T={c.T} Hq={c.Hq} Hkv={c.Hkv} B={c.B} new={c.new_lens.tolist()}")
    prefill_inputs(c.block_tables, c.context_lens, c.query_start, c.T, c.B, c.NB, c.max_query_len)
    return assert_attention_close(run(pa, c), ref(c), c.name)


NEW = [1, 15, 16, 17, 33, 64, 65, 130]
CACHED = [0, 0, 5, 100, 0, 31, 16, 7]


@pytest.mark.parametrize("B", [8, 16, 32, 48])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_ragged_chunks_all_groups_and_block_sizes(pa, G, B):
    c = W.make_prefill_case(f"ragged_G{G}_B{B}", 3000 + 10 * G + B, NEW, CACHED,
                            Hq=2 * G, Hkv=2, B=B)
    check(pa, c)


@pytest.mark.parametrize("n", [63, 64, 65, 127, 128, 129, 255, 257])
def test_prompt_lengths_around_workgroup_row_blocks(pa, n):
    # one head: a workgroup covers 64 rows (4 waves of 16) in the default build,
    # 128 with two row tiles per wave; these lengths straddle both edges
    c = W.make_prefill_case(f"prompt_{n}", 3100 + n, [n, 3], [0, 40], Hq=1, Hkv=1, B=16)
    check(pa, c)


def test_chunked_prefill_is_bit_identical_to_one_pass(pa):
    # the rows of a second chunk (first 200 tokens cached) equal the same rows
    # of a single pass over all 333: per row the arithmetic depends only on the
    # row's position, not on which rows share its wave or workgroup
    full = W.make_prefill_case("one_pass", 3200, [333], [0], Hq=8, Hkv=2, B=16)
    one = run(pa, full)
    chunk = W.PrefillCase(name="second_chunk", seed=3200, S=1, Hq=8, Hkv=2, D=full.D, B=16,
                          NB=full.NB, context_lens=full.context_lens,
                          new_lens=np.array([133], np.int32),
                          query_start=np.array([0, 133], np.int32),
                          block_tables=full.block_tables, query=full.query[200:].copy(),
                          k_pool=full.k_pool, v_pool=full.v_pool, scale=full.scale)
    two = run(pa, chunk)
    assert np.array_equal(u16(two), u16(one[200:]))
    assert_attention_close(two, ref(chunk), "second_chunk")


def test_relabelling_physical_blocks_is_bit_identical(pa):
    c = W.make_prefill_case("relabel", 3300, [70, 200, 9], [30, 0, 300], Hq=4, Hkv=4, B=16)
    base = run(pa, c)
    rng = np.random.default_rng(3301)
    perm = rng.permutation(c.NB)
    inv = np.argsort(perm)           # new id of old block b is inv[b]
    kp = c.k_pool[perm]
    vp = c.v_pool[perm]
    tables = np.where(c.block_tables >= 0, inv[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    again = run(pa, c, kp, vp, tables)
    assert np.array_equal(u16(again), u16(base))


@pytest.mark.parametrize("poison", [np.float16(np.nan), np.float16(np.inf)])
@pytest.mark.parametrize("B", [32, 8])
def test_unused_slots_and_blocks_never_reach_the_output(pa, poison, B):
    c = W.make_prefill_case(f"poison_B{B}", 3400 + (B == 8), [40, 77], [3, 0], Hq=4, Hkv=2, B=B)
    clean = run(pa, c)
    kp, vp = c.k_pool.copy(), c.v_pool.copy()
    used = np.zeros(c.NB, bool)
    for s in range(c.S):
        L = int(c.context_lens[s])
        ids = c.block_tables[s, :oracle.blocks_for(L, c.B)]
        used[ids] = True
        tail = L % c.B
        if tail:
            kp[ids[-1], :, tail:, :] = poison
            vp[ids[-1], :, tail:, :] = poison
    kp[~used] = poison
    vp[~used] = poison
    dirty = run(pa, c, kp, vp)
    assert np.array_equal(u16(dirty), u16(clean))


def relayout(c, B):
    """The same logical keys and values in a fresh pool of block size B (blocks
    handed out in order), with the case's queries."""
    rows = [oracle.blocks_for(int(L), B) for L in c.context_lens]
    NB = sum(rows) + 1
    tables = np.full((c.S, max(rows)), -1, np.int32)
    kp = np.zeros((NB, c.Hkv, B, c.D), np.float16)
    vp = np.zeros_like(kp)
    nxt = 0
    for s, L in enumerate(c.context_lens.tolist()):
        K = oracle.gather(c.k_pool, c.block_tables[s], L, c.B)
        V = oracle.gather(c.v_pool, c.block_tables[s], L, c.B)
        for j in range(rows[s]):
            tables[s, j] = nxt
            n = min(B, L - j * B)
            kp[nxt, :, :n] = K[:, j * B:j * B + n]
            vp[nxt, :, :n] = V[:, j * B:j * B + n]
            nxt += 1
    return W.PrefillCase(**{**c.__dict__, "name": f"{c.name}_as_B{B}", "B": B, "NB": NB,
                            "block_tables": tables, "k_pool": kp, "v_pool": vp})


@pytest.mark.parametrize("G", [1, 4])
def test_block_size_8_is_bit_identical_to_16(pa, G):
    # a 16-token unit of the kernel is then two blocks; the staged keys and
    # values, and so every output bit, are those of the same tokens at B = 16
    c16 = W.make_prefill_case(f"b8_vs_b16_G{G}", 3450 + G, [1, 9, 16, 40, 77, 130],
                              [0, 8, 7, 16, 3, 100], Hq=2 * G, Hkv=2, B=16)
    c8 = relayout(c16, 8)
    check(pa, c16)
    check(pa, c8)
    assert np.array_equal(u16(run(pa, c8)), u16(run(pa, c16)))


def test_empty_and_out_of_range_sequences_leave_their_rows_alone(pa):
    c = W.make_prefill_case("empty", 3500, [20, 0, 35], [10, 50, 0], Hq=2, Hkv=2, B=16)
    sentinel = np.full(c.query.shape, np.float16(7.0))
    got = run(pa, c, out=sentinel)
    assert_attention_close(got, ref(c), "empty")
    # a sequence whose query range leaves [0, T] is skipped entirely
    bad = W.PrefillCase(**{**c.__dict__, "query_start": np.array([0, 20, 20, 99], np.int32)})
    got = run(pa, bad, out=sentinel, max_query_len=35)
    assert_attention_close(got[:20], ref(c)[:20], "bad range: first sequence")
    assert np.all(got[20:] == np.float16(7.0))


def test_rows_before_position_zero_are_zero(pa):
    # n > L is a caller error the kernel contains: rows whose position would be
    # negative come out as zeros, the others as for the last L rows alone
    c = W.make_prefill_case("n_gt_L", 3600, [24], [0], Hq=2, Hkv=2, B=16)
    over = W.PrefillCase(**{**c.__dict__, "context_lens": np.array([20], np.int32)})
    got = run(pa, over)
    assert np.all(got[:4] == 0)
    fit = W.PrefillCase(**{**c.__dict__, "context_lens": np.array([20], np.int32),
                           "new_lens": np.array([20], np.int32),
                           "query_start": np.array([0, 20], np.int32),
                           "query": c.query[4:].copy()})
    assert_attention_close(got[4:], ref(fit), "n_gt_L tail")


def test_shared_prefix_flow_copy_write_prefill(pa):
    """64 sequences share a cached 500-token prompt (grouped heads 32/8): each
    takes a private copy of the partly filled block, its suffix is stored with
    pa_write_kv and processed by one pa_prefill. Pools are compared bit for bit
    with the oracle's own copy and write, outputs within tolerance."""
    d = W.prefix_prefill()
    S, B = d["S"], d["B"]
    seq = np.concatenate([np.full(n, s, np.int32) for s, n in enumerate(d["new_lens"])])
    pos = np.concatenate([np.arange(d["prefix_len"], L, dtype=np.int32) for L in d["context_lens"]])
    ks, vs = np.concatenate(d["suffix_k"]), np.concatenate(d["suffix_v"])
    say("prefix_prefill", f"S={S} T={len(seq)} NB={d['NB']}")
    kp, vp = dev(d["k_pool"]), dev(d["v_pool"])
    pa.pa_copy_blocks(kp, vp, dev(d["copy_pairs"]))
    t = dev(d["tables"])
    slots = pa.pa_slot_mapping(t, B, d["NB"], seq_ids=dev(seq), positions=dev(pos))
    pa.pa_write_kv(dev(ks), dev(vs), kp, vp, slots)
    out = pa.pa_prefill(dev(d["prefill_query"]), kp, vp, t, dev(d["context_lens"]),
                        dev(d["query_start"]), int(d["new_lens"].max()), d["scale"])
    got = host(out)
    rk, rv = oracle.copy_blocks(d["k_pool"], d["v_pool"], d["copy_pairs"])
    rslots = oracle.token_slots(d["tables"], seq, pos, B, d["NB"])
    assert np.array_equal(host(slots), rslots)
    rk, rv = oracle.write_kv(rk, rv, ks, vs, rslots)
    assert np.array_equal(u16(host(kp)), u16(rk)) and np.array_equal(u16(host(vp)), u16(rv))
    want = oracle.prefill(d["prefill_query"], rk, rv, d["tables"], d["context_lens"],
                          d["query_start"], d["scale"])
    assert_attention_close(got, want, "prefix_prefill")


def test_chat_prefill_full_size_every_row(pa):
    """The benchmark's batch (16 prompts of 100-2000 tokens, 32 heads, B = 16)
    in its launch configuration: every row, head and dimension of the output
    against the oracle."""
    c = W.chat_prefill()
    say(c.name, f"T={c.T} NB={c.NB}")
    got = run(pa, c)
    assert_attention_close(got, ref(c), c.name)


def test_long_prompt_after_long_cached_prefix_sampled(pa):
    """6,000 new tokens after 3,000 cached ones (282 blocks of 32, many LDS
    chunks and table reads per row block), grouped heads 4/2; sampled rows
    across the whole chunk against the oracle's attention."""
    c = W.make_prefill_case("long_prompt", 3700, [6000], [3000], Hq=4, Hkv=2, B=32)
    say(c.name, f"T={c.T} L={int(c.context_lens[0])} NB={c.NB}")
    got = run(pa, c)
    L, n = int(c.context_lens[0]), int(c.new_lens[0])
    K = oracle.gather(c.k_pool, c.block_tables[0], L, c.B)
    V = oracle.gather(c.v_pool, c.block_tables[0], L, c.B)
    rows = [0, 1, 63, 64, 2047, 2048, 4095, 5000, n - 2, n - 1]
    want = np.empty((len(rows), c.Hq, c.D))
    for i, j in enumerate(rows):
        p = L - n + j
        for h in range(c.Hq):
            g = h // (c.Hq // c.Hkv)
            want[i, h] = oracle.attend(c.query[j, h], K[g, :p + 1], V[g, :p + 1], c.scale)
    assert_attention_close(got[rows], want, c.name)


@pytest.mark.parametrize("G", [1, 4])
def test_many_short_chunks(pa, G):
    # 300 sequences of 1-40 new tokens after cached prefixes of 0-600: many
    # small work items (one row block each) spread over the XCD ranges
    rng = np.random.default_rng(3500 + G)
    new = [int(x) for x in rng.integers(1, 41, 300)]
    cached = [int(x) for x in rng.integers(0, 601, 300)]
    c = W.make_prefill_case(f"short_chunks_G{G}", 3510 + G, new, cached, Hq=2 * G, Hkv=2, B=16)
    check(pa, c)


def test_one_new_token_per_sequence_is_decode(pa):
    # prefill with a single new token per sequence attends exactly like decode
    # over the same cache (the new token at position L - 1)
    rng = np.random.default_rng(3520)
    cached = [int(x) for x in rng.integers(0, 900, 200)]
    c = W.make_prefill_case("one_token_each", 3521, [1] * 200, cached, Hq=8, Hkv=2, B=16)
    check(pa, c)
    dec = oracle.decode(c.query, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale)
    assert_attention_close(run(pa, c), dec, "prefill of one token against decode")
