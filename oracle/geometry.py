"""Block geometry and token-to-slot translation (oracle; test infrastructure only).

[L] = "Paged Attention: OS-Inspired Memory Management for KV Caches".

A pool holds NB physical blocks of B token slots each. Slot numbers run over
the whole pool, block by block: slot = physical_block * B + offset. A
sequence's block table row maps its logical block i (tokens i*B .. i*B+B-1) to
a physical block ([L], "What PagedAttention is"); token t therefore lives in
logical block t // B at offset t % B ([L], listing paged_vs_contiguous.py,
which translates token 37 this way).
"""
from __future__ import annotations

import numpy as np


def blocks_for(L: int, B: int) -> int:
    """Blocks a sequence of L tokens occupies: the smallest n with n * B >= L.

    [L], "How PagedAttention works", step 1: a prompt takes just enough blocks.
    Written as a loop-free integer ceiling; L = 0 needs no block.
    """
    L, B = int(L), int(B)
    if B <= 0 or L < 0:
        raise ValueError("need B > 0 and L >= 0")
    n = L // B
    if n * B < L:
        n += 1
    return n


def logical_block(t: int, B: int) -> int:
    """Index into the table row of the block that holds token t ([L], "What PagedAttention is")."""
    return int(t) // int(B)


def block_offset(t: int, B: int) -> int:
    """Slot of token t inside its block."""
    return int(t) % int(B)


def slot_of(table_row, t: int, B: int) -> int:
    """Pool-wide slot of token t: physical block times B plus the offset.

    [L], listing paged_vs_contiguous.py: the table entry of logical block
    t // B is the physical block.
    """
    return int(table_row[logical_block(t, B)]) * int(B) + block_offset(t, B)


def empty_slots(L: int, B: int) -> int:
    """Unfilled slots in the last block ([L], "Worked example, step by step")."""
    return blocks_for(L, B) * int(B) - int(L)


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """One token's cache entry: a key and a value vector per layer and KV head
    ([L], "Quick recap: the KV cache")."""
    return 2 * int(layers) * int(kv_heads) * int(head_dim) * int(elem_bytes)


def contiguous_waste(lengths, max_len: int) -> float:
    """Fraction of reserved slots left unused when each request reserves max_len."""
    lengths = [int(x) for x in lengths]
    reserved = max_len * len(lengths)
    return 1.0 - sum(lengths) / reserved


def paged_waste(lengths, B: int) -> float:
    """Fraction of allocated slots left unused when requests take whole blocks."""
    lengths = [int(x) for x in lengths]
    allocated = sum(blocks_for(L, B) for L in lengths) * B
    return 1.0 - sum(lengths) / allocated


def _checked_slot(tables, s: int, t: int, B: int, NB: int) -> int:
    """slot_of with the library's rule for bad inputs: -1 when the position is
    negative, past the row, or the entry is not a block of the pool."""
    MB = tables.shape[1]
    if t < 0:
        return -1
    j = logical_block(t, B)
    if j >= MB:
        return -1
    phys = int(tables[s, j])
    if phys < 0 or phys >= NB:
        return -1
    return slot_of(tables[s], t, B)


def decode_slots(tables, context_lens, B: int, NB: int) -> np.ndarray:
    """Slot of each sequence's newest token, position L - 1 (int64 [S]).

    The context length counts the token being decoded, so its key and value
    are stored at position L - 1 before attention reads the cache ([L], "How
    PagedAttention works", step 2: a new token fills the next slot of the
    last block). -1 for L <= 0 and for positions the table cannot place.
    """
    tables = np.asarray(tables)
    out = np.empty(len(context_lens), dtype=np.int64)
    for s, L in enumerate(context_lens):
        out[s] = _checked_slot(tables, s, int(L) - 1, B, NB)
    return out


def token_slots(tables, seq_ids, positions, B: int, NB: int) -> np.ndarray:
    """Slots of arbitrary (sequence, position) tokens, int64 [T]; -1 where the
    table cannot place the token."""
    tables = np.asarray(tables)
    out = np.empty(len(positions), dtype=np.int64)
    for i, (s, t) in enumerate(zip(seq_ids, positions)):
        s = int(s)
        out[i] = -1 if not (0 <= s < tables.shape[0]) else _checked_slot(tables, s, int(t), B, NB)
    return out
