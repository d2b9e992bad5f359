"""Parity of decode when the batch's work is split evenly over the resident
workgroups (any group size, once sequences span more than one partition; the
vector kernel for groups of 1 and 2 query heads, the matrix-core kernel for 4
and 8). Runs of equal length then start and end anywhere inside
a sequence and may cover several (sequence, KV head) pairs, so these cases aim
at the run boundaries: empty sequences between others, sequences of one unit,
one long sequence among many short ones (many pieces for one sequence), and
back-to-back calls that reuse one workspace. Each case checks on the host that
the split is engaged (its workspace size) before comparing with the oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_attention_close, dev, host, pa_module, say
from host_validate import decode_inputs
from decode_rules import even_split

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def pa():
    return pa_module()


def kv_heads(G, few):
    """KV heads for a case: `few` for groups of 4 and 8; for one or two query
    heads per KV head 64, so that the small batches here still have more
    partitions than one round of the vector kernel's resident workgroups, the
    size from which that kernel takes the split."""
    return few if G >= 4 else 64


def split_engaged(pa, c, P):
    Pc = pa.pa_decode_partition_size(c.S, c.Hq, c.Hkv, c.B, c.max_context_len, P)
    parts = -(-c.max_context_len // Pc)
    return even_split(c.S, c.Hq, c.Hkv, Pc, parts), parts


def run_and_check(pa, c, P, workspace=None, expect_split=True):
    engaged, parts = split_engaged(pa, c, P)
    assert engaged == expect_split, (c.name, parts)
    want_ws = c.S * c.Hq * (parts + engaged) * (D + 2) * 4 + engaged * c.S * c.Hkv * 4
    assert pa.pa_decode_workspace_bytes(c.S, c.Hq, c.Hkv, D, c.B, c.max_context_len, P) == want_ws
    say(c.name, f"S={c.S} Hq={c.Hq} Hkv={c.Hkv} B={c.B} P={P} parts={parts} even={engaged}")
    decode_inputs(c.block_tables, c.context_lens, c.B, c.NB, c.max_context_len)
    out = pa.pa_decode(dev(c.query), dev(c.k_pool), dev(c.v_pool), dev(c.block_tables),
                       dev(c.context_lens), c.max_context_len, c.scale, partition_size=P,
                       workspace=workspace)
    got = host(out)
    ref = oracle.decode(c.query, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale)
    assert_attention_close(got, ref, c.name)
    empty = c.context_lens == 0
    assert not got[empty].any()
    return got


@pytest.mark.parametrize("B", [8, 16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("P", [16, 64, 256])
def test_mixed_lengths_with_empty_sequences(pa, G, B, P):
    lens = [0, 1, 15, 16, 17, P - 1, P, P + 1, 0, 3 * P + 5, 40, 0, 700, 1, 2 * P]
    lens = [max(0, L) for L in lens]
    Hkv = kv_heads(G, 4)
    c = W.make_case(f"even_G{G}_B{B}_P{P}", 6000 + G + B + P, lens, Hq=Hkv * G, Hkv=Hkv, B=B)
    run_and_check(pa, c, P)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_one_long_sequence_among_many_short(pa, G):
    # the long sequence is cut into many pieces, short ones share runs
    lens = [20] * 60 + [5000] + [33] * 40
    c = W.make_case(f"even_long_short_G{G}", 6100 + G, lens, Hq=2 * G, Hkv=2, B=16)
    run_and_check(pa, c, 64)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_eight_kv_heads_across_xcds(pa, G):
    # 8 KV heads: each XCD's eighth of the runs is about one head
    rng = np.random.default_rng(61 + G)
    lens = rng.integers(0, 900, size=96)
    c = W.make_case(f"even_h8_G{G}", 6200 + G, lens, Hq=8 * G, Hkv=8, B=16)
    run_and_check(pa, c, 128)


def test_more_than_1024_sequences_use_one_workgroup_per_partition(pa):
    lens = np.full(1025, 40, np.int32)
    lens[::7] = 17
    c = W.make_case("even_over_1024", 6300, lens, Hq=4, Hkv=1, B=16)
    run_and_check(pa, c, 16, expect_split=False)


def test_back_to_back_calls_share_one_workspace(pa):
    import torch
    big = W.make_case("even_ws_big", 6400, [900, 0, 333, 1500, 17, 64], Hq=32, Hkv=8, B=16)
    small = W.make_case("even_ws_small", 6401, [100, 250, 0, 70], Hq=32, Hkv=8, B=16)
    need = pa.pa_decode_workspace_bytes(big.S, big.Hq, big.Hkv, D, 16, big.max_context_len, 64)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)   # no part of the workspace needs to start at a particular value
    a1 = run_and_check(pa, big, 64, workspace=ws)
    run_and_check(pa, small, 64, workspace=ws)
    a2 = run_and_check(pa, big, 64, workspace=ws)
    assert np.array_equal(a1.view(np.uint16), a2.view(np.uint16))


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_relabelling_physical_blocks_is_bit_identical_under_the_split(pa, G):
    Hkv = kv_heads(G, 4)
    c = W.make_case(f"even_relabel_G{G}", 6500 + G, [700, 90, 1023, 5, 2000, 0, 1200],
                    Hq=Hkv * G, Hkv=Hkv, B=16)
    engaged, _ = split_engaged(pa, c, 256)
    assert engaged
    say(c.name, "relabel")
    base = host(pa.pa_decode(dev(c.query), dev(c.k_pool), dev(c.v_pool), dev(c.block_tables),
                             dev(c.context_lens), c.max_context_len, c.scale, partition_size=256))
    perm = np.random.default_rng(98).permutation(c.NB).astype(np.int32)
    tables = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    inv = np.argsort(perm)
    kp, vp = c.k_pool[inv], c.v_pool[inv]
    got = host(pa.pa_decode(dev(c.query), dev(kp), dev(vp), dev(tables), dev(c.context_lens),
                            c.max_context_len, c.scale, partition_size=256))
    assert np.array_equal(base.view(np.uint16), got.view(np.uint16))


@pytest.mark.parametrize("Hq", [8, 16, 32, 64])
def test_chat_lengths_grouped_heads_full_size_every_output(pa, Hq):
    """Layer 0 of the batch-128 chat lengths with 8 KV heads (groups of 1, 2,
    4 and 8) in the benchmark's launch configuration, which takes the even
    split: every (sequence, head, dimension) of the output against the
    oracle."""
    c = W.chat_layer(0, Hq=Hq, Hkv=8)
    engaged, parts = split_engaged(pa, c, 0)
    assert engaged and parts == 3, parts
    say(c.name, f"NB={c.NB} maxL={c.max_context_len} even split")
    kp, vp = W.device_pools(c.NB, c.Hkv, c.B, c.D, seed=W.chat_pool_seed(0))
    out = pa.pa_decode(dev(c.query), kp, vp, dev(c.block_tables), dev(c.context_lens),
                       c.max_context_len, c.scale)
    got = host(out)
    k_host, v_host = host(kp), host(vp)
    del kp, vp
    ref = oracle.decode(c.query, k_host, v_host, c.block_tables, c.context_lens, c.scale)
    assert_attention_close(got, ref, c.name)


@pytest.mark.parametrize("seed", range(10))
def test_random_even_split_shapes(pa, seed):
    # batches up to the split's 1,024-sequence limit (16 chunks of lengths per
    # wave), every block size the kernels specialise, partitions of 16 to 1,024
    # tokens, lengths with zeros and unit edges
    rng = np.random.default_rng(6700 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.choice([8, 16, 32, 48]))
    S = int(rng.choice([3, 65, 300, 1024])) if seed % 3 else 1024
    top = 160 if S >= 300 else 1800
    lens = rng.integers(0, top, size=S).astype(np.int32)
    lens[rng.random(S) < 0.1] = 0
    edge = rng.random(S) < 0.1
    lens[edge] = rng.choice([1, 15, 16, 17, 31, 33], size=int(edge.sum()))
    lens[int(rng.integers(0, S))] = top           # the longest sets the partitions
    P = int(rng.choice([16, 64])) if top < 1000 else int(rng.choice([0, 64, 1024]))
    c = W.make_case(f"even_rand_{seed}", 6800 + seed, lens, Hq=G * Hkv, Hkv=Hkv, B=B)
    engaged, _ = split_engaged(pa, c, P)
    if not engaged:
        pytest.skip("this draw gives one partition per sequence")
    run_and_check(pa, c, P)
