"""Cache contents: gather through a table, token writes, block copies
(oracle; test infrastructure only).

[L] = "Paged Attention: OS-Inspired Memory Management for KV Caches";
[B] = "What is PagedAttention and how does it manage KV cache?".

Pool layout: [NB, Hkv, B, D]. Inside one physical block and one KV head the B
tokens sit one after another, each a row of D values ([B], "How PagedAttention
works": tokens are contiguous within a block).
"""
from __future__ import annotations

import numpy as np

from .geometry import blocks_for


def gather(pool: np.ndarray, table_row, L: int, B: int) -> np.ndarray:
    """The sequence's first L tokens, in logical order, as [Hkv, L, D].

    Reads the blocks the table names in table order ([L], "How PagedAttention
    works", step 4: walk the table and load each block), lays them end to end
    and keeps the first L token rows.
    """
    NB, Hkv, Bp, D = pool.shape
    if Bp != B:
        raise ValueError("block size mismatch")
    n = blocks_for(L, B)
    ids = np.asarray(table_row[:n], dtype=np.int64)
    if len(ids) < n:
        raise ValueError("table row shorter than the context needs")
    if n and (ids.min() < 0 or ids.max() >= NB):
        raise ValueError("table entry outside the pool")
    out = np.empty((Hkv, n * B, D), dtype=pool.dtype)
    for i, b in enumerate(ids):
        out[:, i * B:(i + 1) * B, :] = pool[b]
    return out[:, :L, :]


def write_kv(k_pool, v_pool, key, value, slot_mapping):
    """Store token i's key/value rows ([Hkv, D]) at slot_mapping[i] in both pools.

    Returns new pools; the inputs are not modified. A negative slot means the
    token is not stored, and so does a slot past the pool's last slot (the
    library skips such writes rather than touch memory outside the pool).
    Two tokens aimed at one slot is a caller error and is rejected here.
    ([L], "How PagedAttention works", step 2: a new token goes into the next
    free slot of the last block, no allocation.)
    """
    k_out, v_out = k_pool.copy(), v_pool.copy()
    NB, Hkv, B, D = k_pool.shape
    slots = np.asarray(slot_mapping, dtype=np.int64)
    valid = [int(x) for x in slots if 0 <= x < NB * B]
    if len(valid) != len(set(valid)):
        raise ValueError("duplicate slots in one write")
    for i, slot in enumerate(slots):
        slot = int(slot)
        if slot < 0 or slot >= NB * B:
            continue
        blk, off = divmod(slot, B)
        k_out[blk, :, off, :] = key[i]
        v_out[blk, :, off, :] = value[i]
    return k_out, v_out


def copy_blocks(k_pool, v_pool, pairs):
    """For each (src, dst): physical block dst becomes a copy of block src, in
    both pools, all heads and all B slots.

    Every source is read as it was before the call. Destinations must be
    distinct and must not be sources (caller error otherwise); a pair naming a
    block outside the pool is skipped, as the library does.
    ([L], "Memory sharing across requests": copy-on-write gives the writer a
    private copy of a shared block.)
    """
    k_out, v_out = k_pool.copy(), v_pool.copy()
    NB = k_pool.shape[0]
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    ok = [(int(s), int(d)) for s, d in pairs if 0 <= s < NB and 0 <= d < NB]
    dsts = [d for _, d in ok]
    if len(dsts) != len(set(dsts)) or set(dsts) & {s for s, _ in ok}:
        raise ValueError("copy destinations must be distinct and not sources")
    for src, dst in ok:
        k_out[dst] = k_pool[src]
        v_out[dst] = v_pool[src]
    return k_out, v_out


def swap_blocks(dst_k, dst_v, src_k, src_v, pairs):
    """For each (src, dst): block dst of the destination pools becomes a copy
    of block src of the source pools (both pools, all heads, all B slots).

    Returns new destination pools. Pairs naming a block outside either pool
    are skipped; destinations must be distinct. ([L], "Memory sharing across
    requests" and [B], "Why it matters for KV cache": blocks evicted to host
    memory under pressure and fetched back when the request resumes.)
    """
    k_out, v_out = dst_k.copy(), dst_v.copy()
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    ok = [(int(s), int(d)) for s, d in pairs
          if 0 <= s < src_k.shape[0] and 0 <= d < dst_k.shape[0]]
    dsts = [d for _, d in ok]
    if len(dsts) != len(set(dsts)):
        raise ValueError("swap destinations must be distinct")
    for s_, d in ok:
        k_out[d] = src_k[s_]
        v_out[d] = src_v[s_]
    return k_out, v_out
