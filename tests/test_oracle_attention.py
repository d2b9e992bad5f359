"""Pins for the oracle's paged decode attention.

Independent references: closed forms, torch's CPU scaled_dot_product_attention
in fp64 (its own softmax and its own grouped-query head mapping), brute force
over every table on tiny pools, and the pages' statement that paging does not
change the result.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from conftest import load_golden


def place(Kc, table, B, NB, fill=0.0):
    """Test-side layout of contiguous [H, L, D] tokens into a pool through a table."""
    H, L, D = Kc.shape
    pool = np.full((NB, H, B, D), fill, dtype=Kc.dtype)
    for t in range(L):
        pool[table[t // B], :, t % B, :] = Kc[:, t, :]
    return pool


def sdpa(q, K, V, scale):
    """torch reference: q [Hq, D], K/V [Hkv, L, D] -> [Hq, D] in fp64."""
    qt = torch.tensor(np.asarray(q, np.float64))[None, :, None, :]
    kt = torch.tensor(np.asarray(K, np.float64))[None]
    vt = torch.tensor(np.asarray(V, np.float64))[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
    return o[0, :, 0, :].numpy()


def one_seq(q, Kc, Vc, B, table, NB, scale):
    kp, vp = place(Kc, table, B, NB), place(Vc, table, B, NB)
    tables = np.full((1, max(len(table), 1)), -1, dtype=np.int32)
    tables[0, :len(table)] = table
    return oracle.decode(q[None], kp, vp, tables, np.array([Kc.shape[1]]), scale)[0]


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((2, 8)).astype(np.float16)
    K = rng.standard_normal((2, 1, 8)).astype(np.float16)
    V = rng.standard_normal((2, 1, 8)).astype(np.float16)
    out = one_seq(q, K, V, 4, [3], 5, 0.3)
    assert np.array_equal(out, V[:, 0, :].astype(np.float64))


@pytest.mark.parametrize("case", ["zero_query", "equal_keys"])
def test_uniform_weights_give_the_mean_value(case):
    rng = np.random.default_rng(1)
    H, L, D, B = 2, 13, 16, 4
    q = rng.standard_normal((H, D))
    K = rng.standard_normal((H, L, D))
    V = rng.standard_normal((H, L, D))
    if case == "zero_query":
        q[:] = 0
    else:
        K[:] = K[:, :1, :]
    table = rng.permutation(8)[:4]
    out = one_seq(q, K, V, B, table, 8, 1 / math.sqrt(D))
    assert np.allclose(out, V.mean(axis=1), rtol=0, atol=1e-13)


def test_constant_values_give_that_constant():
    rng = np.random.default_rng(2)
    H, L, D = 3, 21, 8
    q = rng.standard_normal((H, D))
    K = rng.standard_normal((H, L, D)) * 3
    V = np.broadcast_to(rng.standard_normal((H, 1, D)), (H, L, D)).copy()
    out = one_seq(q, K, V, 8, [2, 0, 5], 6, 0.7)
    assert np.allclose(out, V[:, 0, :], rtol=0, atol=1e-13)


def test_two_tokens_hand_computed():
    # q = e0, K0 = 2 e0, K1 = 0, scale 1/2 -> scores 1 and 0
    D = 4
    q = np.zeros((1, D)); q[0, 0] = 1
    K = np.zeros((1, 2, D)); K[0, 0, 0] = 2
    V = np.array([[[1.0, 2, 3, 4], [5.0, 6, 7, 8]]])
    out = one_seq(q, K, V, 1, [1, 0], 2, 0.5)
    w0 = math.e / (1 + math.e)
    assert np.allclose(out[0], w0 * V[0, 0] + (1 - w0) * V[0, 1], rtol=0, atol=1e-14)


def test_dominant_key_with_huge_scores_stays_finite():
    # scores near 1e4: exp overflows unless the maximum is subtracted first
    rng = np.random.default_rng(3)
    H, L, D = 1, 9, 8
    q = np.ones((H, D))
    K = rng.standard_normal((H, L, D))
    K[0, 6] = 1250.0          # score 1e4 at scale 1
    K[0, 2] = 1249.0          # score 9992: weight e^-8 relative
    V = rng.standard_normal((H, L, D))
    out = one_seq(q, K, V, 4, [0, 1, 2], 3, 1.0)
    w = 1 / (1 + math.exp(-8))
    assert np.all(np.isfinite(out))
    assert np.allclose(out[0], w * V[0, 6] + (1 - w) * V[0, 2], atol=1e-6)


def test_grouped_query_heads_read_kv_head_h_div_group():
    rng = np.random.default_rng(4)
    Hq, Hkv, L, D = 8, 2, 10, 4
    q = rng.standard_normal((Hq, D))
    K = rng.standard_normal((Hkv, L, D))
    V = np.zeros((Hkv, L, D))
    V[0] = 1.0
    V[1] = 2.0
    out = one_seq(q, K, V, 4, [1, 3, 0], 4, 0.5)
    assert np.allclose(out[:4], 1.0) and np.allclose(out[4:], 2.0)


def test_matches_torch_sdpa_on_contiguous_tokens():
    rng = np.random.default_rng(5)
    for Hq, Hkv, L, B in [(4, 4, 40, 16), (32, 8, 77, 16), (6, 2, 33, 32), (2, 1, 1, 16)]:
        D = 128
        q = rng.standard_normal((Hq, D)).astype(np.float16)
        K = rng.standard_normal((Hkv, L, D)).astype(np.float16)
        V = rng.standard_normal((Hkv, L, D)).astype(np.float16)
        nb = oracle.blocks_for(L, B)
        NB = nb + 3
        table = rng.permutation(NB)[:nb]
        out = one_seq(q, K, V, B, table, NB, 1 / math.sqrt(D))
        ref = sdpa(q, K, V, 1 / math.sqrt(D))
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_unused_slots_and_blocks_never_reach_the_output():
    rng = np.random.default_rng(6)
    H, L, D, B, NB = 2, 19, 8, 4, 9
    q = rng.standard_normal((H, D))
    K = rng.standard_normal((H, L, D))
    V = rng.standard_normal((H, L, D))
    table = np.array([4, 0, 7, 2, 5])
    clean = one_seq(q, K, V, B, table, NB, 0.4)
    for poison in (np.nan, np.inf, -np.inf):
        kp = place(K, table, B, NB, fill=poison)
        vp = place(V, table, B, NB, fill=poison)
        tables = np.array([list(table) + [-1, -1]], dtype=np.int32)
        out = oracle.decode(q[None], kp, vp, tables, np.array([L]), 0.4)[0]
        assert np.array_equal(out, clean)


def test_output_is_invariant_under_relabelling_physical_blocks():
    rng = np.random.default_rng(7)
    H, L, D, B, NB = 2, 30, 16, 4, 12
    q = rng.standard_normal((H, D))
    K = rng.standard_normal((H, L, D))
    V = rng.standard_normal((H, L, D))
    nb = oracle.blocks_for(L, B)
    base = one_seq(q, K, V, B, np.arange(nb), NB, 0.25)
    for _ in range(5):
        table = rng.permutation(NB)[:nb]
        assert np.array_equal(one_seq(q, K, V, B, table, NB, 0.25), base)


@pytest.mark.parametrize("B,Lmax", [(1, 4), (2, 8), (4, 8)])
def test_brute_force_every_table_equals_contiguous(B, Lmax):
    rng = np.random.default_rng(8 + B)
    H, D = 2, 4
    for L in range(1, Lmax + 1):
        q = rng.standard_normal((H, D))
        K = rng.standard_normal((H, L, D))
        V = rng.standard_normal((H, L, D))
        ref = sdpa(q, K, V, 0.5)
        nb = oracle.blocks_for(L, B)
        NB = nb + 2
        for table in itertools.permutations(range(NB), nb):
            out = one_seq(q, K, V, B, list(table), NB, 0.5)
            assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_lifecycle_table_walk_equals_contiguous_attention():
    g = load_golden("lifecycle.json")
    rng = np.random.default_rng(9)
    H, D, B, L = 4, 128, g["block"], 49
    q = rng.standard_normal((H, D)).astype(np.float16)
    K = rng.standard_normal((H, L, D)).astype(np.float16)
    V = rng.standard_normal((H, L, D)).astype(np.float16)
    out = one_seq(q, K, V, B, g["table_walk"], 16, 1 / math.sqrt(D))
    assert np.allclose(out, sdpa(q, K, V, 1 / math.sqrt(D)), rtol=1e-12, atol=1e-13)


def test_partition_merge_identity():
    rng = np.random.default_rng(10)
    D, L = 32, 97
    q = rng.standard_normal(D)
    K = rng.standard_normal((L, D)) * 2
    V = rng.standard_normal((L, D))
    full = oracle.attend(q, K, V, 0.3)
    for _ in range(20):
        cuts = np.sort(rng.choice(np.arange(1, L), size=rng.integers(1, 8), replace=False))
        edges = [0, *cuts.tolist(), L]
        parts = [oracle.attend_partial(q, K[a:b], V[a:b], 0.3) for a, b in zip(edges, edges[1:])]
        parts.append(oracle.attend_partial(q, K[:0], V[:0], 0.3))   # an empty partition
        assert np.allclose(oracle.merge_partials(parts), full, rtol=0, atol=1e-12)


def test_zero_length_gives_zero_output_and_bad_lengths_raise():
    q = np.ones((1, 2, 4), dtype=np.float16)
    pool = np.ones((2, 2, 4, 4), dtype=np.float16)
    tables = np.array([[1]], dtype=np.int32)
    assert not oracle.decode(q, pool, pool, tables, np.array([0]), 1.0).any()
    with pytest.raises(ValueError):
        oracle.decode(q, pool, pool, tables, np.array([5]), 1.0)


# ---------------------------------------------------------------------------
# prefill: a chunk of new tokens per sequence, causal, through the table
# ---------------------------------------------------------------------------

def _prefill_case(rng, lens, nq, Hq, Hkv, B, D=16, extra_blocks=3):
    S = len(lens)
    MB = max(oracle.blocks_for(L, B) for L in lens)
    NB = sum(oracle.blocks_for(L, B) for L in lens) + extra_blocks
    perm = rng.permutation(NB)
    tables = np.full((S, MB), -1, np.int32)
    off = 0
    for s, L in enumerate(lens):
        n = oracle.blocks_for(L, B)
        tables[s, :n] = perm[off:off + n]
        off += n
    kp = rng.standard_normal((NB, Hkv, B, D))
    vp = rng.standard_normal((NB, Hkv, B, D))
    qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), Hq, D))
    return q, kp, vp, tables, np.array(lens, np.int32), qs


def test_prefill_of_one_token_is_decode():
    rng = np.random.default_rng(20)
    q, kp, vp, t, L, qs = _prefill_case(rng, [17, 40, 5], [1, 1, 1], 4, 2, 4)
    # prefill works on all rows of a sequence at once, decode on one query:
    # the same sums in another order, equal to rounding
    assert np.allclose(oracle.prefill(q, kp, vp, t, L, qs, 0.3), oracle.decode(q, kp, vp, t, L, 0.3),
                       rtol=1e-13, atol=1e-15)


def test_prompt_prefill_equals_causal_sdpa():
    rng = np.random.default_rng(21)
    for Hq, Hkv, L, B in [(4, 4, 37, 4), (8, 2, 50, 16), (2, 1, 1, 4)]:
        q, kp, vp, t, lens, qs = _prefill_case(rng, [L], [L], Hq, Hkv, B)
        got = oracle.prefill(q, kp, vp, t, lens, qs, 0.25)
        K = oracle.gather(kp, t[0], L, B)
        V = oracle.gather(vp, t[0], L, B)
        qt = torch.tensor(q.transpose(1, 0, 2))[None]
        ref = F.scaled_dot_product_attention(qt, torch.tensor(K)[None], torch.tensor(V)[None],
                                             scale=0.25, is_causal=True, enable_gqa=True)
        assert np.allclose(got, ref[0].numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-13)


def test_chunked_prefill_rows_match_full_prefill():
    # the second chunk, with the first already cached, gives the same rows as one pass
    rng = np.random.default_rng(22)
    q, kp, vp, t, lens, qs = _prefill_case(rng, [45], [45], 4, 4, 8)
    full = oracle.prefill(q, kp, vp, t, lens, qs, 0.4)
    tail = oracle.prefill(q[30:], kp, vp, t, lens, np.array([0, 15]), 0.4)
    assert np.allclose(tail, full[30:], rtol=1e-13, atol=1e-15)


def test_prefill_last_row_sees_everything_first_row_sees_the_prefix():
    rng = np.random.default_rng(23)
    q, kp, vp, t, lens, qs = _prefill_case(rng, [30], [6], 2, 2, 4)
    out = oracle.prefill(q, kp, vp, t, lens, qs, 0.5)
    K = oracle.gather(kp, t[0], 30, 4)
    V = oracle.gather(vp, t[0], 30, 4)
    assert np.allclose(out[5, 1], oracle.attend(q[5, 1], K[1], V[1], 0.5), rtol=0, atol=1e-14)
    assert np.allclose(out[0, 0], oracle.attend(q[0, 0], K[0, :25], V[0, :25], 0.5), rtol=0, atol=1e-14)


def test_prefill_brute_force_tables_and_poison():
    rng = np.random.default_rng(24)
    B, L, Hq, Hkv, D = 2, 5, 2, 1, 4
    q = rng.standard_normal((3, Hq, D))
    K = rng.standard_normal((Hkv, L, D))
    V = rng.standard_normal((Hkv, L, D))
    qt = torch.tensor(q.transpose(1, 0, 2))[None]
    mask = torch.ones(3, L, dtype=torch.bool).tril(diagonal=L - 3)
    ref = F.scaled_dot_product_attention(qt, torch.tensor(K)[None], torch.tensor(V)[None],
                                         attn_mask=mask, scale=0.7, enable_gqa=True)[0].numpy()
    nb = oracle.blocks_for(L, B)
    for table in itertools.permutations(range(nb + 2), nb):
        kp = place(K, table, B, nb + 2, fill=np.nan)
        vp = place(V, table, B, nb + 2, fill=np.nan)
        out = oracle.prefill(q, kp, vp, np.array([table]), np.array([L]), np.array([0, 3]), 0.7)
        assert np.allclose(out, ref.transpose(1, 0, 2), rtol=1e-12, atol=1e-14)


def test_causal_attention_rows_are_attend_over_their_prefix():
    # row i of a causal block is plain attention over keys 0 .. first + i
    rng = np.random.default_rng(25)
    Q = rng.standard_normal((6, 8))
    K = rng.standard_normal((11, 8))
    V = rng.standard_normal((11, 8))
    out = oracle.causal_attention(Q, K, V, 5, 0.6)
    for i in range(6):
        ref = oracle.attend(Q[i], K[:6 + i], V[:6 + i], 0.6)
        assert np.allclose(out[i], ref, rtol=1e-13, atol=1e-15)
    with pytest.raises(ValueError):
        oracle.causal_attention(Q, K, V, 6, 0.6)     # the last row would sit past the keys
