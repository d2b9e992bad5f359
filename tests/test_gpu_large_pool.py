"""Pools larger than 4 GiB: every kernel addresses blocks with 64-bit offsets.

K and V pools of 147,456 blocks x 8 KV heads x 16 tokens x 128 dims fp16 (4.5 GiB
each) live on the device. Only the blocks that three sequences use are filled
(seeded), most of them past the 4 GiB boundary and a few just below it; the rest
of the pools is never written. The oracle runs on a compact copy that holds just
those blocks, with the tables renumbered. One decode step is checked end to end:
slot mapping (bit-exact), pa_write_kv (bit-exact on every used block),
pa_copy_blocks into two blocks past the boundary (bit-exact), pa_decode, and
pa_prefill over the last tokens of each sequence (both within the attention
tolerance)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_attention_close, dev, host, pa_module, say, u16
from host_validate import copy_pairs, decode_inputs, prefill_inputs, write_batch

pytestmark = pytest.mark.gpu

HKV, HQ, B, D = 8, 32, 16, 128
BLOCK_BYTES = HKV * B * D * 2             # 32 KiB per block, all KV heads
HIGH = (1 << 32) // BLOCK_BYTES           # first block whose offset is 4 GiB or more
NB = HIGH + HIGH // 8                     # 4.5 GiB per pool


@pytest.fixture(scope="module")
def pa():
    return pa_module()


def test_pools_beyond_4_gib(pa):
    import torch
    rng = np.random.default_rng(9100)
    cached = np.array([299, 516, 39], np.int32)          # tokens already in the cache
    lens = cached + 1                                      # after this step's new token
    S = len(lens)
    rows = [oracle.blocks_for(int(L), B) for L in lens]
    n_used = sum(rows)
    # physical ids: a few just below the boundary, the rest above it
    ids = np.concatenate([rng.choice(np.arange(HIGH - 4, HIGH), 2, replace=False),
                          rng.choice(np.arange(HIGH, NB), n_used - 2, replace=False)])
    ids = rng.permutation(ids).astype(np.int64)
    tables = np.full((S, max(rows) + 1), -1, np.int32)
    compact = np.full_like(tables, -1)
    k = 0
    for s, r in enumerate(rows):
        tables[s, :r] = ids[k:k + r]
        compact[s, :r] = np.arange(k, k + r)
        k += r
    say("pools_beyond_4_gib", f"NB={NB} (first block past 4 GiB: {HIGH}) used={n_used} "
        f"max id={int(ids.max())} lens={lens.tolist()}")
    decode_inputs(tables, lens, B, NB, int(lens.max()))

    ck = W.f16_normal(rng, (n_used, HKV, B, D))
    cv = W.f16_normal(rng, (n_used, HKV, B, D))
    kp = torch.empty((NB, HKV, B, D), dtype=torch.float16, device="cuda")
    vp = torch.empty_like(kp)
    idx = torch.from_numpy(ids).cuda()
    kp.index_copy_(0, idx, dev(ck))
    vp.index_copy_(0, idx, dev(cv))

    # slot mapping and the new tokens' writes
    key = W.f16_normal(rng, (S, HKV, D))
    value = W.f16_normal(rng, (S, HKV, D))
    t_dev, l_dev = dev(tables), dev(lens)
    slots = pa.pa_slot_mapping(t_dev, B, NB, context_lens=l_dev)
    want_slots = oracle.decode_slots(tables, lens, B, NB)
    assert np.array_equal(host(slots), want_slots)
    assert (want_slots // B >= HIGH).any()                 # some writes land past 4 GiB
    write_batch(want_slots, B, NB)
    pa.pa_write_kv(dev(key), dev(value), kp, vp, slots)
    ck, cv = oracle.write_kv(ck, cv, key, value, oracle.decode_slots(compact, lens, B, n_used))
    assert np.array_equal(u16(host(kp.index_select(0, idx))), u16(ck))
    assert np.array_equal(u16(host(vp.index_select(0, idx))), u16(cv))

    # copy-on-write into two unused blocks past the boundary
    free = np.setdiff1d(np.arange(HIGH, NB), ids)
    pairs = np.array([[ids[0], free[-1]], [ids[-1], free[0]]], np.int32)
    copy_pairs(pairs, NB)
    pa.pa_copy_blocks(kp, vp, dev(pairs))
    for src, dst in pairs.tolist():
        assert np.array_equal(u16(host(kp[dst])), u16(host(kp[src])))
        assert np.array_equal(u16(host(vp[dst])), u16(host(vp[src])))
    assert np.array_equal(u16(host(kp.index_select(0, idx))), u16(ck))   # sources unchanged

    # one decode step through the table
    q = W.f16_normal(rng, (S, HQ, D))
    scale = 1.0 / np.sqrt(D)
    out = pa.pa_decode(dev(q), kp, vp, t_dev, l_dev, int(lens.max()), scale)
    assert_attention_close(host(out), oracle.decode(q, ck, cv, compact, lens, scale),
                           "decode beyond 4 GiB")

    # prefill over the last n tokens of each sequence
    n = np.array([5, 17, 1], np.int32)
    qs = np.zeros(S + 1, np.int32)
    qs[1:] = np.cumsum(n)
    query = W.f16_normal(rng, (int(qs[-1]), HQ, D))
    prefill_inputs(tables, lens, qs, int(qs[-1]), B, NB, int(n.max()))
    got = pa.pa_prefill(dev(query), kp, vp, t_dev, l_dev, dev(qs), int(n.max()), scale)
    assert_attention_close(host(got), oracle.prefill(query, ck, cv, compact, lens, qs, scale),
                           "prefill beyond 4 GiB")
    del kp, vp
    torch.cuda.empty_cache()
