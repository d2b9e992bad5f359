"""Seeded random sweep of decode and prefill shapes against the oracle: batch
size, grouped-query size, block size, partition size and lengths (zero,
block and unit edges, cached prefixes) drawn per seed, every output element
within the attention tolerance. Complements the hand-picked edge cases."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_attention_close, dev, host, pa_module, say
from host_validate import decode_inputs, prefill_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return pa_module()


def draw_lengths(rng, S, B, top):
    pool = [0, 1, B - 1 if B > 1 else 1, B, B + 1, 15, 16, 17, 31, 33]
    out = [int(rng.choice(pool)) if rng.random() < 0.4 else int(rng.integers(1, top)) for _ in range(S)]
    return [max(x, 0) for x in out]


@pytest.mark.parametrize("seed", range(12))
def test_random_decode_shapes(pa, seed):
    rng = np.random.default_rng(7100 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.choice([8, 16, 32, 48, 64]))
    S = int(rng.integers(1, 20))
    lens = draw_lengths(rng, S, B, 1500)
    if max(lens) == 0:
        lens[0] = 1
    P = int(rng.choice([0, 16, 64, 256, 1024]))
    c = W.make_case(f"rand_decode_{seed}", 7200 + seed, lens, Hq=G * Hkv, Hkv=Hkv, B=B)
    say(c.name, f"S={S} G={G} Hkv={Hkv} B={B} P={P} lens={lens}")
    decode_inputs(c.block_tables, c.context_lens, c.B, c.NB, c.max_context_len)
    kp, vp = dev(c.k_pool), dev(c.v_pool)
    tables, L = dev(c.block_tables), dev(c.context_lens)
    slots = pa.pa_slot_mapping(tables, c.B, c.NB, context_lens=L)
    pa.pa_write_kv(dev(c.key_new), dev(c.value_new), kp, vp, slots)
    got = host(pa.pa_decode(dev(c.query), kp, vp, tables, L, c.max_context_len, c.scale,
                            partition_size=P))
    rs = oracle.decode_slots(c.block_tables, c.context_lens, c.B, c.NB)
    assert np.array_equal(host(slots), rs)
    rk, rv = oracle.write_kv(c.k_pool, c.v_pool, c.key_new, c.value_new, rs)
    ref = oracle.decode(c.query, rk, rv, c.block_tables, c.context_lens, c.scale)
    assert_attention_close(got, ref, c.name)


@pytest.mark.parametrize("seed", range(10))
def test_random_prefill_shapes(pa, seed):
    rng = np.random.default_rng(7300 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2]))
    B = int(rng.choice([8, 16, 32, 48, 64]))
    S = int(rng.integers(1, 8))
    new = [int(x) for x in rng.integers(0, 300, S)]
    new = [int(rng.choice([1, 15, 16, 17, 63, 64, 65])) if rng.random() < 0.3 else x for x in new]
    if max(new) == 0:
        new[0] = 5
    cached = [int(rng.choice([0, 0, 1, 31, 200, 517])) for _ in range(S)]
    c = W.make_prefill_case(f"rand_prefill_{seed}", 7400 + seed, new, cached, Hq=G * Hkv, Hkv=Hkv, B=B)
    say(c.name, f"S={S} G={G} Hkv={Hkv} B={B} new={new} cached={cached}")
    prefill_inputs(c.block_tables, c.context_lens, c.query_start, c.T, c.B, c.NB, c.max_query_len)
    got = host(pa.pa_prefill(dev(c.query), dev(c.k_pool), dev(c.v_pool), dev(c.block_tables),
                             dev(c.context_lens), dev(c.query_start), c.max_query_len, c.scale))
    ref = oracle.prefill(c.query, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                         c.query_start, c.scale)
    assert_attention_close(got, ref, c.name)


@pytest.mark.parametrize("seed", range(10))
def test_random_decode_odd_kv_head_counts(pa, seed):
    # KV head counts that are not powers of two (3, 5, 6, 7, 12): the walk over
    # (KV head, sequence) pairs, the XCD-contiguous work order and the
    # partition grid take any count; batches up to 40 sequences and short
    # partitions put groups of 1 and 2 past the even split's threshold too
    rng = np.random.default_rng(7500 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([3, 5, 6, 7, 12]))
    B = int(rng.choice([8, 16, 32]))
    S = int(rng.integers(2, 41))
    lens = draw_lengths(rng, S, B, 1500)
    if max(lens) == 0:
        lens[0] = 1
    P = int(rng.choice([0, 64, 256]))
    c = W.make_case(f"rand_decode_kv{Hkv}_{seed}", 7600 + seed, lens, Hq=G * Hkv, Hkv=Hkv, B=B)
    say(c.name, f"S={S} G={G} Hkv={Hkv} B={B} P={P} max_len={max(lens)}")
    decode_inputs(c.block_tables, c.context_lens, c.B, c.NB, c.max_context_len)
    got = host(pa.pa_decode(dev(c.query), dev(c.k_pool), dev(c.v_pool), dev(c.block_tables),
                            dev(c.context_lens), c.max_context_len, c.scale, partition_size=P))
    ref = oracle.decode(c.query, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale)
    assert_attention_close(got, ref, c.name)


@pytest.mark.parametrize("seed", range(6))
def test_random_prefill_odd_kv_head_counts(pa, seed):
    rng = np.random.default_rng(7700 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([3, 5, 6]))
    B = int(rng.choice([8, 16, 32]))
    S = int(rng.integers(1, 6))
    new = [int(x) for x in rng.integers(1, 300, S)]
    cached = [int(rng.choice([0, 17, 200])) for _ in range(S)]
    c = W.make_prefill_case(f"rand_prefill_kv{Hkv}_{seed}", 7800 + seed, new, cached, Hq=G * Hkv,
                            Hkv=Hkv, B=B)
    say(c.name, f"S={S} G={G} Hkv={Hkv} B={B} new={new} cached={cached}")
    prefill_inputs(c.block_tables, c.context_lens, c.query_start, c.T, c.B, c.NB, c.max_query_len)
    got = host(pa.pa_prefill(dev(c.query), dev(c.k_pool), dev(c.v_pool), dev(c.block_tables),
                             dev(c.context_lens), dev(c.query_start), c.max_query_len, c.scale))
    ref = oracle.prefill(c.query, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                         c.query_start, c.scale)
    assert_attention_close(got, ref, c.name)
