"""Parity of pa_decode (HIP) against the fp64 CPU oracle on the workloads and
edge cases, plus the invariants the pages fix (relabelling and sharing of
physical blocks leave the output unchanged, bit for bit on the GPU)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_attention_close, dev, host, pa_module, say, u16
from host_validate import decode_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return pa_module()


def decode_step(pa, case, kp, vp, partition_size=0):
    """GPU: slot of each new token, store it, decode. Returns (out, slots) on the host."""
    tables, lens = dev(case.block_tables), dev(case.context_lens)
    slots = pa.pa_slot_mapping(tables, case.B, case.NB, context_lens=lens)
    pa.pa_write_kv(dev(case.key_new), dev(case.value_new), kp, vp, slots)
    out = pa.pa_decode(dev(case.query), kp, vp, tables, lens, case.max_context_len, case.scale,
                       partition_size=partition_size)
    return host(out), host(slots)


def oracle_step(case, k_pool, v_pool):
    slots = oracle.decode_slots(case.block_tables, case.context_lens, case.B, case.NB)
    kp, vp = oracle.write_kv(k_pool, v_pool, case.key_new, case.value_new, slots)
    return oracle.decode(case.query, kp, vp, case.block_tables, case.context_lens, case.scale), slots


def check_case(pa, case, partition_size=0):
    say(case.name, f"S={case.S} Hq={case.Hq} Hkv={case.Hkv} B={case.B} P={partition_size}")
    decode_inputs(case.block_tables, case.context_lens, case.B, case.NB, case.max_context_len)
    kp, vp = dev(case.k_pool), dev(case.v_pool)
    got, slots = decode_step(pa, case, kp, vp, partition_size)
    ref, ref_slots = oracle_step(case, case.k_pool, case.v_pool)
    assert np.array_equal(slots, ref_slots)
    return assert_attention_close(got, ref, case.name)


def test_tiny_worked_example(pa):
    check_case(pa, W.tiny_worked_example())


def test_lifecycle_growth_walk(pa):
    g = W.growth_example()
    kp, vp = dev(g["k_pool"]), dev(g["v_pool"])
    say("growth walk 7-2-9-4, L=49")
    table = dev(g["table_after"])
    slots = pa.pa_slot_mapping(table, g["B"], g["NB"], seq_ids=dev(np.zeros(9, np.int32)),
                               positions=dev(g["positions"]))
    pa.pa_write_kv(dev(g["new_k"]), dev(g["new_v"]), kp, vp, slots)
    lens = np.array([g["len_after"]], dtype=np.int32)
    out = host(pa.pa_decode(dev(g["query"]), kp, vp, table, dev(lens), 49, g["scale"]))
    rslots = oracle.token_slots(g["table_after"], np.zeros(9, int), g["positions"], g["B"], g["NB"])
    rk, rv = oracle.write_kv(g["k_pool"], g["v_pool"], g["new_k"], g["new_v"], rslots)
    assert np.array_equal(u16(host(kp)), u16(rk)) and np.array_equal(u16(host(vp)), u16(rv))
    ref = oracle.decode(g["query"], rk, rv, g["table_after"], lens, g["scale"])
    assert_attention_close(out, ref, "growth")


def test_seven_b_single_layer(pa):
    check_case(pa, W.seven_b_single_layer())


@pytest.mark.parametrize("P", [16, 64, 256, 512, 1024])
def test_seven_b_partition_sweep(pa, P):
    check_case(pa, W.seven_b_single_layer(), partition_size=P)


def test_long_context_b32(pa):
    c = W.long_context(with_pools=False)
    say(c.name, "device pools")
    kp, vp = W.device_pools(c.NB, c.Hkv, c.B, c.D, seed=c.seed * 1000)
    c.k_pool, c.v_pool = host(kp), host(vp)
    ref, _ = oracle_step(c, c.k_pool, c.v_pool)
    for P in (0, 512, 1024):          # 512: 8 partitions per sequence
        kp2, vp2 = kp.clone(), vp.clone()
        say(c.name, f"P={P}")
        got, _ = decode_step(pa, c, kp2, vp2, P)
        assert_attention_close(got, ref, f"long_context P={P}")


def _shared_prefix_inputs():
    d = W.shared_prefix()
    case = W.DecodeCase(name="shared_prefix", seed=4, S=d["S"], Hq=d["Hq"], Hkv=d["Hkv"], D=d["D"],
                        B=d["B"], NB=d["NB"], context_lens=d["context_lens"],
                        block_tables=d["tables"], query=d["query"],
                        key_new=np.stack([k[-1] for k in d["suffix_k"]]),
                        value_new=np.stack([v[-1] for v in d["suffix_v"]]),
                        k_pool=d["k_pool"], v_pool=d["v_pool"], scale=d["scale"])
    # setup writes: positions prefix_len .. L-2 of every sequence
    seq, pos, ks, vs = [], [], [], []
    for s in range(d["S"]):
        n = int(d["context_lens"][s]) - d["prefix_len"] - 1
        seq += [s] * n
        pos += list(range(d["prefix_len"], d["prefix_len"] + n))
        ks.append(d["suffix_k"][s][:-1])
        vs.append(d["suffix_v"][s][:-1])
    return d, case, np.array(seq, np.int32), np.array(pos, np.int32), np.concatenate(ks), np.concatenate(vs)


def _run_shared(pa, d, case, seq, pos, ks, vs, tables, k_pool, v_pool, pairs):
    kp, vp = dev(k_pool), dev(v_pool)
    if len(pairs):
        pa.pa_copy_blocks(kp, vp, dev(pairs))
    t = dev(tables)
    slots = pa.pa_slot_mapping(t, case.B, kp.shape[0], seq_ids=dev(seq), positions=dev(pos))
    pa.pa_write_kv(dev(ks), dev(vs), kp, vp, slots)
    lens = dev(case.context_lens)
    new_slots = pa.pa_slot_mapping(t, case.B, kp.shape[0], context_lens=lens)
    pa.pa_write_kv(dev(case.key_new), dev(case.value_new), kp, vp, new_slots)
    out = pa.pa_decode(dev(case.query), kp, vp, t, lens, case.max_context_len, case.scale)
    return host(out), kp, vp, host(slots)


def test_shared_prefix_gqa_and_private_twin_bit_identical(pa):
    d, case, seq, pos, ks, vs = _shared_prefix_inputs()
    say("shared_prefix: copy-on-write, suffix writes, decode (G=4)")
    out, kp, vp, slots = _run_shared(pa, d, case, seq, pos, ks, vs, d["tables"], d["k_pool"],
                                     d["v_pool"], d["copy_pairs"])
    # oracle: same three steps
    rk, rv = oracle.copy_blocks(d["k_pool"], d["v_pool"], d["copy_pairs"])
    rslots = oracle.token_slots(d["tables"], seq, pos, case.B, case.NB)
    assert np.array_equal(slots, rslots)
    rk, rv = oracle.write_kv(rk, rv, ks, vs, rslots)
    ref, _ = oracle_step(case, rk, rv)
    assert_attention_close(out, ref, "shared_prefix")

    # twin: every sequence holds private copies of the 31 full prompt blocks
    S, NB = case.S, case.NB
    n_full = d["prefix_len"] // case.B
    extra = S * n_full
    k2 = np.concatenate([d["k_pool"], np.zeros((extra,) + d["k_pool"].shape[1:], np.float16)])
    v2 = np.concatenate([d["v_pool"], np.zeros((extra,) + d["v_pool"].shape[1:], np.float16)])
    tables2 = d["tables"].copy()
    pairs2 = [tuple(p) for p in d["copy_pairs"]]
    for s in range(S):
        for j in range(n_full):
            new_id = NB + s * n_full + j
            pairs2.append((int(d["shared_ids"][j]), new_id))
            tables2[s, j] = new_id
    say("shared_prefix twin with private prefix copies")
    out2, _, _, _ = _run_shared(pa, d, case, seq, pos, ks, vs, tables2, k2, v2,
                                np.array(pairs2, np.int32))
    assert np.array_equal(u16(out), u16(out2))


def relabelled(c, seed):
    """The same case with every physical block id permuted."""
    perm = np.random.default_rng(seed).permutation(c.NB)   # new id of old block b is perm[b]
    k2 = np.empty_like(c.k_pool)
    v2 = np.empty_like(c.v_pool)
    k2[perm] = c.k_pool
    v2[perm] = c.v_pool
    t2 = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    return W.DecodeCase(**{**c.__dict__, "block_tables": t2, "k_pool": k2, "v_pool": v2})


def poisoned_pools(c, poison):
    """Pools with every slot that is not one of the sequences' first L tokens
    (the slot this step writes included) set to poison."""
    keep = np.zeros(c.NB * c.B, bool)
    for s, L in enumerate(c.context_lens):
        for t in range(int(L)):
            keep[oracle.slot_of(c.block_tables[s], t, c.B)] = True
    kp, vp = c.k_pool.copy(), c.v_pool.copy()
    mask = ~keep.reshape(c.NB, c.B)
    kp.transpose(0, 2, 1, 3)[mask] = poison
    vp.transpose(0, 2, 1, 3)[mask] = poison
    return kp, vp


def test_relabelling_physical_blocks_is_bit_identical(pa):
    c = W.seven_b_single_layer()
    say("relabel physical ids")
    base, _ = decode_step(pa, c, dev(c.k_pool), dev(c.v_pool))
    c2 = relabelled(c, 99)
    got, _ = decode_step(pa, c2, dev(c2.k_pool), dev(c2.v_pool))
    assert np.array_equal(u16(base), u16(got))


@pytest.mark.parametrize("poison", [np.float16(np.nan), np.float16(np.inf), np.float16(-np.inf)])
def test_unused_slots_and_blocks_never_reach_the_output(pa, poison):
    c = W.make_case("poison", 31, [1, 15, 16, 17, 33, 200, 511, 513], Hq=8, Hkv=4, B=16)
    clean, _ = decode_step(pa, c, dev(c.k_pool), dev(c.v_pool), partition_size=64)
    kp, vp = poisoned_pools(c, poison)
    say(f"poison {poison}")
    got, _ = decode_step(pa, c, dev(kp), dev(vp), partition_size=64)
    assert np.array_equal(u16(clean), u16(got))


# Groups of 4 and 8 query heads run on the matrix cores: the edge cases and
# invariants again for that kernel (at B = 8 each 16-token unit reads two blocks).

@pytest.mark.parametrize("B", [8, 16, 32, 48])
@pytest.mark.parametrize("G", [4, 8])
def test_mfma_groups_lengths_partitions_and_table_chunks(pa, G, B):
    # empty sequences, partial units, partitions starting inside blocks, the
    # reduce, and single partitions longer than 64 blocks (several table chunks)
    lens = [0, 1, 15, 16, 17, 100, 1025, 64 * B + 17, 2 * 64 * 16 + 5]
    c = W.make_case(f"group{G}_B{B}", 5000 + 10 * G + B, lens, Hq=2 * G, Hkv=2, B=B)
    for ps in (0, 48, 1040, 4096):
        check_case(pa, c, partition_size=ps)


@pytest.mark.parametrize("B", [8, 16, 32])
@pytest.mark.parametrize("G", [4, 8])
@pytest.mark.parametrize("poison", [np.float16(np.nan), np.float16(np.inf), np.float16(-np.inf)])
def test_mfma_groups_unused_slots_and_blocks_never_reach_the_output(pa, poison, G, B):
    c = W.make_case(f"group{G}_poison_B{B}", 5100 + 10 * G + B, [1, 15, 16, 17, 33, 200, 511, 513],
                    Hq=2 * G, Hkv=2, B=B)
    clean, _ = decode_step(pa, c, dev(c.k_pool), dev(c.v_pool), partition_size=64)
    kp, vp = poisoned_pools(c, poison)
    say(f"group of {G}, B={B}, poison {poison}")
    got, _ = decode_step(pa, c, dev(kp), dev(vp), partition_size=64)
    assert np.array_equal(u16(clean), u16(got))


@pytest.mark.parametrize("G", [4, 8])
def test_mfma_groups_relabelling_physical_blocks_is_bit_identical(pa, G):
    c = W.make_case(f"group{G}_relabel", 5200 + G, [700, 90, 1023, 5, 2000], Hq=8 * G, Hkv=8, B=16)
    say(f"group of {G}: relabel physical ids")
    base, _ = decode_step(pa, c, dev(c.k_pool), dev(c.v_pool))
    c2 = relabelled(c, 98)
    got, _ = decode_step(pa, c2, dev(c2.k_pool), dev(c2.v_pool))
    assert np.array_equal(u16(base), u16(got))
    ref, _ = oracle_step(c, c.k_pool, c.v_pool)
    assert_attention_close(base, ref, c.name)


EDGE_B16 = [1, 15, 16, 17, 63, 64, 65, 128, 131]


@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_edge_lengths_all_groups(pa, B, G):
    P = 4 * B
    lens = sorted({1, B - 1, B, B + 1, P - 1, P, P + 1, 2 * P + 3, 5 * B + 7})
    c = W.make_case(f"edges_B{B}_G{G}", 1000 + B + G, lens, Hq=2 * G, Hkv=2, B=B)
    for ps in (0, P, B):
        check_case(pa, c, partition_size=ps)


def test_partition_at_least_context_equals_single_pass(pa):
    c = W.make_case("single_pass", 41, [700, 90, 1023], Hq=4, Hkv=4, B=16)
    say("single pass vs P >= L")
    a, _ = decode_step(pa, c, dev(c.k_pool), dev(c.v_pool), partition_size=1024)
    b, _ = decode_step(pa, c, dev(c.k_pool), dev(c.v_pool), partition_size=2048)
    assert np.array_equal(u16(a), u16(b))
    ref, _ = oracle_step(c, c.k_pool, c.v_pool)
    assert_attention_close(a, ref, "single_pass")


def test_long_partitions_over_64_blocks(pa):
    # partitions longer than 64 blocks walk the table in several chunks
    c = W.make_case("long_partition", 42, [2000, 1025, 64 * 16 + 1], Hq=2, Hkv=1, B=16)
    check_case(pa, c, partition_size=2048)
    check_case(pa, c, partition_size=1040)


def test_zero_length_gives_zeros(pa):
    c = W.make_case("zero_len", 43, [0, 5, 0, 40], Hq=4, Hkv=4, B=16)
    say("zero lengths")
    kp, vp = dev(c.k_pool), dev(c.v_pool)
    tables, lens = dev(c.block_tables), dev(c.context_lens)
    out = host(pa.pa_decode(dev(c.query), kp, vp, tables, lens, 40, c.scale, partition_size=16))
    ref = oracle.decode(c.query, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale)
    assert not out[0].any() and not out[2].any()
    assert_attention_close(out, ref, "zero_len")


def test_repeat_runs_are_bit_identical(pa):
    c = W.seven_b_single_layer()
    tables, lens, q = dev(c.block_tables), dev(c.context_lens), dev(c.query)
    kp, vp = dev(c.k_pool), dev(c.v_pool)
    say("determinism")
    a = host(pa.pa_decode(q, kp, vp, tables, lens, c.max_context_len, c.scale))
    b = host(pa.pa_decode(q, kp, vp, tables, lens, c.max_context_len, c.scale))
    assert np.array_equal(u16(a), u16(b))


def test_device_errors_are_reported(pa):
    import torch
    c = W.tiny_worked_example()
    with pytest.raises(pa.PaError, match="PA_ERR_WORKSPACE"):
        pa.pa_decode(dev(c.query), dev(c.k_pool), dev(c.v_pool), dev(c.block_tables),
                     dev(c.context_lens), 48, c.scale, partition_size=16,
                     workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(pa.PaError, match="PA_ERR_UNSUPPORTED"):
        q = torch.zeros((2, 4, 64), dtype=torch.float16, device="cuda")
        pool = torch.zeros((16, 4, 16, 64), dtype=torch.float16, device="cuda")
        pa.pa_decode(q, pool, pool, dev(c.block_tables), dev(c.context_lens), 48, 0.1)


def test_chat_batch128_full_size_every_output(pa):
    """Full-size layers 0 and 31 of the batch-128 chat workload in the
    benchmark's launch configuration (default partition size): every slot
    checked bit-exactly, every (sequence, head, dimension) of the output
    against the oracle, which gets the pools as they were before the step and
    performs its own write of the new tokens."""
    lengths = W.chat_lengths()
    for layer in (0, W.CHAT_LAYERS - 1):
        c = W.chat_layer(layer, lengths=lengths)
        say(c.name, f"NB={c.NB} maxL={c.max_context_len}")
        kp, vp = W.device_pools(c.NB, c.Hkv, c.B, c.D, seed=W.chat_pool_seed(layer))
        k_before, v_before = host(kp), host(vp)
        got, slots = decode_step(pa, c, kp, vp)
        del kp, vp
        ref_slots = oracle.decode_slots(c.block_tables, c.context_lens, c.B, c.NB)
        assert np.array_equal(slots, ref_slots)
        rk, rv = oracle.write_kv(k_before, v_before, c.key_new, c.value_new, ref_slots)
        del k_before, v_before
        ref = oracle.decode(c.query, rk, rv, c.block_tables, c.context_lens, c.scale)
        del rk, rv
        assert_attention_close(got, ref, c.name)


@pytest.mark.parametrize("B", [48, 64, 128, 256])
@pytest.mark.parametrize("G", [1, 4])
def test_other_block_sizes_and_partitions_inside_blocks(pa, B, G):
    lens = [1, 15, B - 1, B, B + 17, 3 * B + 5, 700]
    c = W.make_case(f"B{B}_G{G}", 2000 + B + G, lens, Hq=2 * G, Hkv=2, B=B)
    for ps in (0, 16, 48, 2 * B, 1024):
        check_case(pa, c, partition_size=ps)



B8_LENS = [1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 129, 1030]


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_block_size_8_units_spanning_two_blocks(pa, G):
    """B = 8: every 16-token work unit reads two blocks; lengths end in either
    half of a unit, and partitions of 16 to 2048 tokens (over 64 blocks: two
    table chunks) start on unit boundaries."""
    c = W.make_case(f"B8_G{G}", 2200 + G, B8_LENS, Hq=2 * G, Hkv=2, B=8)
    for ps in (0, 16, 48, 1024, 2048):
        check_case(pa, c, partition_size=ps)


def relayout(c, B):
    """The same logical keys and values in a fresh pool of block size B (blocks
    handed out in order), with the case's new tokens and queries."""
    S = c.S
    rows = [oracle.blocks_for(int(L), B) for L in c.context_lens]
    NB = sum(rows) + 1
    MB = max(rows)
    tables = np.full((S, MB), -1, np.int32)
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
    return W.DecodeCase(**{**c.__dict__, "B": B, "NB": NB, "block_tables": tables,
                           "k_pool": kp, "v_pool": vp})


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_block_size_8_is_bit_identical_to_16(pa, G):
    # the arithmetic order depends only on logical positions, so the same
    # tokens give the same bits whatever the block size
    c8 = W.make_case(f"B8_vs_16_G{G}", 2300 + G, B8_LENS, Hq=2 * G, Hkv=2, B=8)
    c16 = relayout(c8, 16)
    for ps in (0, 16, 64):
        say(f"B=8 vs B=16, G={G}, P={ps}")
        a, _ = decode_step(pa, c8, dev(c8.k_pool), dev(c8.v_pool), partition_size=ps)
        b, _ = decode_step(pa, c16, dev(c16.k_pool), dev(c16.v_pool), partition_size=ps)
        assert np.array_equal(u16(a), u16(b))


def test_block_size_8_unused_slots_and_blocks_never_reach_the_output(pa):
    c = W.make_case("B8_poison", 2400, B8_LENS, Hq=4, Hkv=2, B=8)
    clean, _ = decode_step(pa, c, dev(c.k_pool), dev(c.v_pool), partition_size=48)
    keep = np.zeros(c.NB * c.B, bool)
    for s, L in enumerate(c.context_lens):
        for t in range(int(L)):
            keep[oracle.slot_of(c.block_tables[s], t, c.B)] = True
    kp, vp = c.k_pool.copy(), c.v_pool.copy()
    mask = ~keep.reshape(c.NB, c.B)
    kp.transpose(0, 2, 1, 3)[mask] = np.float16(np.nan)
    vp.transpose(0, 2, 1, 3)[mask] = np.float16(np.inf)
    say("B=8 poison")
    got, _ = decode_step(pa, c, dev(kp), dev(vp), partition_size=48)
    assert np.array_equal(u16(clean), u16(got))

def test_contiguous_layout_one_block_per_sequence(pa):
    # the pre-paging layout: every sequence in one block as long as the longest
    lens = [1000, 37, 512, 999, 640]
    B = 1008
    c = W.make_case("contiguous", 2100, lens, Hq=8, Hkv=8, B=B)
    assert c.MB == 1
    for ps in (0, 256, 1008):
        check_case(pa, c, partition_size=ps)


def test_very_long_context_65536_tokens(pa):
    """One 65,536-token sequence (4,096 blocks of 16: 64 table windows per
    1,024-token partition sweep, 64 partitions merged) next to a 1-token one."""
    c = W.make_case("ctx65536", 2300, [65536, 1], Hq=4, Hkv=4, B=16)
    say(c.name, f"NB={c.NB} MB={c.MB}")
    for ps in (0, 4096):
        check_case(pa, c, partition_size=ps)
