"""Bit-exact parity of slot translation, token writes and block copies (GPU vs
the CPU oracle), over whole pools compared as uint16."""
import numpy as np
import pytest

import oracle
import workloads as W
from conftest import load_golden
from gpu_util import dev, host, pa_module, say, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    return pa_module()


def test_slot_mapping_decode_form_matches_oracle(pa):
    c = W.seven_b_single_layer()
    say("slot_mapping decode form, 7b_single_layer")
    got = host(pa.pa_slot_mapping(dev(c.block_tables), c.B, c.NB, context_lens=dev(c.context_lens)))
    ref = oracle.decode_slots(c.block_tables, c.context_lens, c.B, c.NB)
    assert got.dtype == np.int64 and np.array_equal(got, ref)


def test_slot_mapping_invalid_inputs_give_minus_one(pa):
    tables = np.array([[3, 1, -1], [0, 2, 5], [7, -1, -1], [1, 9, 2]], dtype=np.int32)
    lens = np.array([5, 12, 0, 6], dtype=np.int32)
    say("slot_mapping invalid inputs")
    got = host(pa.pa_slot_mapping(dev(tables), 4, 8, context_lens=dev(lens)))
    ref = oracle.decode_slots(tables, lens, 4, 8)
    assert np.array_equal(got, ref) and got.tolist() == [4, 23, -1, -1]
    seq = np.array([0, 1, 1, 3, 4, -1, 2], dtype=np.int32)
    pos = np.array([7, 11, 12, 5, 0, 0, 0], dtype=np.int32)
    got = host(pa.pa_slot_mapping(dev(tables), 4, 8, seq_ids=dev(seq), positions=dev(pos)))
    assert np.array_equal(got, oracle.token_slots(tables, seq, pos, 4, 8))


def test_lifecycle_growth_slots(pa):
    g = W.growth_example()
    gold = load_golden("lifecycle.json")
    say("slot_mapping growth walk 7-2-9-4")
    got = host(pa.pa_slot_mapping(dev(g["table_after"]), g["B"], g["NB"],
                                  seq_ids=dev(np.zeros(9, np.int32)),
                                  positions=dev(g["positions"])))
    assert got.tolist() == gold["derived_slots_positions_40_to_48"]


def test_write_kv_bit_exact_whole_pool(pa):
    c = W.seven_b_single_layer()
    kp, vp = dev(c.k_pool), dev(c.v_pool)
    say("write_kv 7b_single_layer")
    slots = pa.pa_slot_mapping(dev(c.block_tables), c.B, c.NB, context_lens=dev(c.context_lens))
    pa.pa_write_kv(dev(c.key_new), dev(c.value_new), kp, vp, slots)
    rk, rv = oracle.write_kv(c.k_pool, c.v_pool, c.key_new, c.value_new, host(slots))
    assert np.array_equal(u16(host(kp)), u16(rk))
    assert np.array_equal(u16(host(vp)), u16(rv))


def test_write_kv_skips_negative_and_out_of_pool_slots(pa):
    rng = np.random.default_rng(21)
    NB, H, B, D, T = 6, 3, 16, 128, 9
    kpool = W.f16_normal(rng, (NB, H, B, D))
    vpool = W.f16_normal(rng, (NB, H, B, D))
    key = W.f16_normal(rng, (T, H, D))
    val = W.f16_normal(rng, (T, H, D))
    slots = np.array([5, -1, 95, 96, 1 << 40, 0, -7, 17, 48], dtype=np.int64)
    kp, vp = dev(kpool), dev(vpool)
    say("write_kv skip rules")
    pa.pa_write_kv(dev(key), dev(val), kp, vp, dev(slots))
    rk, rv = oracle.write_kv(kpool, vpool, key, val, slots)
    assert np.array_equal(u16(host(kp)), u16(rk)) and np.array_equal(u16(host(vp)), u16(rv))


@pytest.mark.parametrize("H,B,D", [(2, 16, 64), (8, 32, 128), (1, 4, 8)])
def test_write_kv_other_shapes(pa, H, B, D):
    rng = np.random.default_rng(H * 100 + B)
    NB = 11
    T = 23
    kpool = W.f16_normal(rng, (NB, H, B, D))
    vpool = W.f16_normal(rng, (NB, H, B, D))
    key = W.f16_normal(rng, (T, H, D))
    val = W.f16_normal(rng, (T, H, D))
    slots = rng.permutation(NB * B)[:T].astype(np.int64)
    kp, vp = dev(kpool), dev(vpool)
    say(f"write_kv H={H} B={B} D={D}")
    pa.pa_write_kv(dev(key), dev(val), kp, vp, dev(slots))
    rk, rv = oracle.write_kv(kpool, vpool, key, val, slots)
    assert np.array_equal(u16(host(kp)), u16(rk)) and np.array_equal(u16(host(vp)), u16(rv))


def test_copy_blocks_shared_prefix_bit_exact(pa):
    d = W.shared_prefix()
    kp, vp = dev(d["k_pool"]), dev(d["v_pool"])
    say("copy_blocks shared_prefix 64 pairs")
    pa.pa_copy_blocks(kp, vp, dev(d["copy_pairs"]))
    rk, rv = oracle.copy_blocks(d["k_pool"], d["v_pool"], d["copy_pairs"])
    assert np.array_equal(u16(host(kp)), u16(rk)) and np.array_equal(u16(host(vp)), u16(rv))


def test_copy_blocks_skips_out_of_pool_pairs_and_large_blocks(pa):
    rng = np.random.default_rng(22)
    NB, H, B, D = 9, 32, 32, 128          # 256 KiB blocks: several workgroups per pair
    kpool = W.f16_normal(rng, (NB, H, B, D))
    vpool = W.f16_normal(rng, (NB, H, B, D))
    pairs = np.array([[0, 3], [1, 9], [-1, 4], [2, 5], [8, 7]], dtype=np.int32)
    kp, vp = dev(kpool), dev(vpool)
    say("copy_blocks skip rules, 256 KiB blocks")
    pa.pa_copy_blocks(kp, vp, dev(pairs))
    rk, rv = oracle.copy_blocks(kpool, vpool, pairs)
    assert np.array_equal(u16(host(kp)), u16(rk)) and np.array_equal(u16(host(vp)), u16(rv))


def test_calls_with_zero_work_are_no_ops(pa):
    import torch
    kp = torch.zeros((2, 1, 16, 128), dtype=torch.float16, device="cuda")
    say("zero-work calls")
    pa.pa_copy_blocks(kp, kp.clone(), torch.zeros((0, 2), dtype=torch.int32, device="cuda"))
    pa.pa_write_kv(torch.zeros((0, 1, 128), dtype=torch.float16, device="cuda"),
                   torch.zeros((0, 1, 128), dtype=torch.float16, device="cuda"), kp, kp.clone(),
                   torch.zeros(0, dtype=torch.int64, device="cuda"))
    assert not host(kp).any()


class Managed:
    """The native block manager with device pools, and the oracle's manager with
    host pools, stepped together: every token's slot and every copy pair of the
    native manager drive pa_copy_blocks and pa_write_kv on the GPU, and must
    equal what the oracle's manager decides for the same step."""

    def __init__(self, pa, rng, NB, H, B, D):
        self.pa, self.rng, self.H, self.D = pa, rng, H, D
        kpool = W.f16_normal(rng, (NB, H, B, D))
        vpool = W.f16_normal(rng, (NB, H, B, D))
        self.kp, self.vp = dev(kpool), dev(vpool)
        self.rk, self.rv = kpool, vpool
        self.nat = pa.BlockManager(NB, B)
        self.ref = oracle.BlockManager(NB, B)

    def step(self, nat_ids, ref_tables):
        """One token for each listed sequence: copies first, then the write."""
        keys = W.f16_normal(self.rng, (len(nat_ids), self.H, self.D))
        vals = W.f16_normal(self.rng, (len(nat_ids), self.H, self.D))
        slots, copies = self.nat.append_tokens(nat_ids)
        c0 = len(self.ref.copies)
        ref_slots = [self.ref.append(t) for t in ref_tables]
        assert slots.tolist() == ref_slots
        assert [tuple(p) for p in copies.tolist()] == self.ref.copies[c0:]
        if len(copies):
            self.pa.pa_copy_blocks(self.kp, self.vp, dev(copies))
            self.rk, self.rv = oracle.copy_blocks(self.rk, self.rv, copies)
        self.pa.pa_write_kv(dev(keys), dev(vals), self.kp, self.vp, dev(slots))
        self.rk, self.rv = oracle.write_kv(self.rk, self.rv, keys, vals, np.array(ref_slots))

    def check_decode(self, nat_ids, ref_tables, MB, what):
        """Pools bit-exact against the oracle, then decode over the sequences."""
        from gpu_util import assert_attention_close
        tables, lens = self.nat.export(nat_ids, MB)
        assert np.array_equal(u16(host(self.kp)), u16(self.rk))
        assert np.array_equal(u16(host(self.vp)), u16(self.rv))
        q = W.f16_normal(self.rng, (len(nat_ids), self.H, self.D))
        out = host(self.pa.pa_decode(dev(q), self.kp, self.vp, dev(tables), dev(lens),
                                     int(lens.max()), 0.088))
        want = oracle.decode(q, self.rk, self.rv,
                             np.array([t.blocks + [-1] * (MB - len(t.blocks)) for t in ref_tables],
                                      np.int32),
                             lens, 0.088)
        assert_attention_close(out, want, what)
        return tables, lens


def test_native_block_manager_drives_the_device_path(pa):
    """Prompt -> fork into samples -> each sample generates tokens, all through
    the native manager (host), whose slots and copy pairs drive pa_copy_blocks,
    pa_write_kv and pa_decode on the GPU. The oracle replays the same steps
    with its own manager, write, copy and decode."""
    m = Managed(pa, np.random.default_rng(77), 96, 4, 16, 128)
    prompt = m.nat.add_sequence()
    rprompt = m.ref.new_sequence()
    say("native manager: 37-token prompt, 5 samples, 21 steps")
    for _ in range(37):
        m.step([prompt], [rprompt])
    samples = [m.nat.fork(prompt) for _ in range(5)]
    rsamples = [m.ref.fork(rprompt) for _ in range(5)]
    m.nat.release(prompt)
    m.ref.free(rprompt)
    for _ in range(21):
        m.step(samples, rsamples)
    _, lens = m.check_decode(samples, rsamples, 6, "managed samples")
    assert (lens == 37 + 21).all()


def test_beam_search_flow_drives_the_device_path(pa):
    """Beam search through the native manager ([L] "Memory sharing across
    requests": candidate beams share their common prefix blocks and diverge at
    the end). A 29-token prompt forks into 4 beams; every step each live beam
    appends a token (a write into a shared partial block copies it first); every
    4 steps beams 1 and 3 are dropped and each survivor forks again. Slots, copy
    pairs, free blocks, the pools and the final decode over the live beams match
    the oracle replaying the same steps, and the prompt's full first block stays
    shared by every live beam."""
    NB = 128
    m = Managed(pa, np.random.default_rng(78), NB, 4, 16, 128)
    prompt = m.nat.add_sequence()
    rprompt = m.ref.new_sequence()
    say("beam search: 29-token prompt, 4 beams, 12 steps, prune and refork every 4")
    for _ in range(29):
        m.step([prompt], [rprompt])
    beams = [m.nat.fork(prompt) for _ in range(4)]
    rbeams = [m.ref.fork(rprompt) for _ in range(4)]
    m.nat.release(prompt)
    m.ref.free(rprompt)
    for t in range(12):
        m.step(beams, rbeams)
        if t % 4 == 3:
            for i in (1, 3):
                m.nat.release(beams[i])
                m.ref.free(rbeams[i])
            beams, rbeams = [beams[0], beams[2]], [rbeams[0], rbeams[2]]
            beams += [m.nat.fork(b) for b in beams]
            rbeams += [m.ref.fork(r) for r in rbeams]
        assert m.nat.num_free() == NB - m.ref.blocks_in_use()
    tables, lens = m.check_decode(beams, rbeams, 4, "beams")
    assert (lens == 29 + 12).all()
    assert len({int(t[0]) for t in tables}) == 1 and m.nat.refcount(int(tables[0][0])) == len(beams)


def test_swap_out_to_pinned_host_and_back_in(pa):
    """Preempt-and-resume: a sequence's blocks go to a pinned host pool and come
    back into other device blocks; the pools match the oracle bit for bit and
    decode on the resumed cache equals decode on the original."""
    import torch
    c = W.seven_b_single_layer()
    kp, vp = dev(c.k_pool), dev(c.v_pool)
    H, B, D = c.Hkv, c.B, c.D
    s = 0                                             # the 853-token sequence
    nb = oracle.blocks_for(int(c.context_lens[s]), B)
    ids = c.block_tables[s, :nb]
    host_k = torch.zeros((nb + 3, H, B, D), dtype=torch.float16).pin_memory()
    host_v = torch.zeros_like(host_k).pin_memory()
    out_pairs = np.stack([ids, np.arange(nb) + 2], 1).astype(np.int32)   # host slots 2..nb+1
    say(f"swap out {nb} blocks to pinned host memory")
    pa.pa_swap_blocks(host_k, host_v, kp, vp, dev(out_pairs))
    torch.cuda.synchronize()
    rk, rv = oracle.swap_blocks(np.zeros((nb + 3, H, B, D), np.float16),
                                np.zeros((nb + 3, H, B, D), np.float16), c.k_pool, c.v_pool, out_pairs)
    assert np.array_equal(u16(host_k.numpy()), u16(rk)) and np.array_equal(u16(host_v.numpy()), u16(rv))

    # resume into a fresh device pool at shuffled positions
    NB2 = nb + 7
    new_ids = np.random.default_rng(5).permutation(NB2)[:nb].astype(np.int32)
    kp2 = torch.full((NB2, H, B, D), float("nan"), dtype=torch.float16, device="cuda")
    vp2 = torch.full_like(kp2, float("nan"))
    in_pairs = np.stack([np.arange(nb) + 2, new_ids], 1).astype(np.int32)
    say("swap back in")
    pa.pa_swap_blocks(kp2, vp2, host_k, host_v, dev(in_pairs))
    lens = c.context_lens[s:s + 1]
    q = dev(c.query[s:s + 1])
    a = host(pa.pa_decode(q, kp, vp, dev(c.block_tables[s:s + 1]), dev(lens), int(lens[0]), c.scale))
    b = host(pa.pa_decode(q, kp2, vp2, dev(new_ids[None, :]), dev(lens), int(lens[0]), c.scale))
    assert np.array_equal(u16(a), u16(b))


def test_swap_refuses_pageable_host_memory(pa):
    import torch
    pool = torch.zeros((4, 1, 16, 128), dtype=torch.float16, device="cuda")
    pageable = torch.zeros((4, 1, 16, 128), dtype=torch.float16)     # not pinned
    pairs = dev(np.array([[0, 1]], np.int32))
    say("swap with pageable memory is refused before any launch")
    with pytest.raises(pa.PaError, match="PA_ERR_UNSUPPORTED"):
        pa.pa_swap_blocks(pageable, pageable, pool, pool, pairs)


def test_append_kv_decode_form_equals_slot_mapping_then_write(pa):
    # one launch against the two calls it replaces and against the oracle:
    # slots and whole pools bit for bit
    c = W.seven_b_single_layer()
    say("append_kv decode form, 7b_single_layer")
    tables, lens = dev(c.block_tables), dev(c.context_lens)
    k_new, v_new = dev(c.key_new), dev(c.value_new)
    kp1, vp1 = dev(c.k_pool), dev(c.v_pool)
    slots1 = pa.pa_slot_mapping(tables, c.B, c.NB, context_lens=lens)
    pa.pa_write_kv(k_new, v_new, kp1, vp1, slots1)
    kp2, vp2 = dev(c.k_pool), dev(c.v_pool)
    import torch
    slots2 = torch.full((c.S,), 77, dtype=torch.int64, device="cuda")
    pa.pa_append_kv(k_new, v_new, kp2, vp2, tables, context_lens=lens, slot_mapping=slots2)
    assert np.array_equal(host(slots1), host(slots2))
    assert np.array_equal(u16(host(kp1)), u16(host(kp2))) and np.array_equal(u16(host(vp1)), u16(host(vp2)))
    ref_slots = oracle.decode_slots(c.block_tables, c.context_lens, c.B, c.NB)
    rk, rv = oracle.write_kv(c.k_pool, c.v_pool, c.key_new, c.value_new, ref_slots)
    assert np.array_equal(host(slots2), ref_slots)
    assert np.array_equal(u16(host(kp2)), u16(rk)) and np.array_equal(u16(host(vp2)), u16(rv))


def test_append_kv_token_form_with_unplaceable_tokens(pa):
    # seq_ids + positions (prefill and extension); tokens whose sequence,
    # position or table entry is out of range get slot -1 and are skipped
    tables = np.array([[3, 1, -1], [0, 2, 5], [7, -1, -1], [1, 9, 2]], dtype=np.int32)
    NB, B, Hkv, D = 8, 4, 2, 16
    seq = np.array([0, 1, 1, 3, 4, -1, 2, 1], dtype=np.int32)
    pos = np.array([7, 11, 12, 5, 0, 0, 0, 3], dtype=np.int32)
    rng = np.random.default_rng(91)
    kp = W.f16_normal(rng, (NB, Hkv, B, D))
    vp = W.f16_normal(rng, (NB, Hkv, B, D))
    key = W.f16_normal(rng, (len(seq), Hkv, D))
    val = W.f16_normal(rng, (len(seq), Hkv, D))
    say("append_kv token form")
    import torch
    gk, gv = dev(kp), dev(vp)
    slots = torch.empty(len(seq), dtype=torch.int64, device="cuda")
    pa.pa_append_kv(dev(key), dev(val), gk, gv, dev(tables), seq_ids=dev(seq), positions=dev(pos),
                    slot_mapping=slots)
    ref_slots = oracle.token_slots(tables, seq, pos, B, NB)
    assert np.array_equal(host(slots), ref_slots)
    rk, rv = oracle.write_kv(kp, vp, key, val, ref_slots)
    assert np.array_equal(u16(host(gk)), u16(rk)) and np.array_equal(u16(host(gv)), u16(rv))
    # without a slot output the pools end the same
    gk2, gv2 = dev(kp), dev(vp)
    pa.pa_append_kv(dev(key), dev(val), gk2, gv2, dev(tables), seq_ids=dev(seq), positions=dev(pos))
    assert np.array_equal(u16(host(gk2)), u16(rk)) and np.array_equal(u16(host(gv2)), u16(rv))
