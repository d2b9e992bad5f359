"""Host validator of the caller's side of the contract (test infrastructure).

The library checks sizes, pointers and alignment on the host. The contents of
the device arrays it is given (block-table entries, context lengths, slots,
copy pairs, query ranges) are the caller's contract: a kernel only contains a
violation (it clamps or skips, so no access leaves the buffers) and the result
is unspecified. These functions check that contract on host copies of the
arrays, so that a test can assert that what it feeds the GPU is valid input,
and that a planted mistake is caught. Each raises InvalidInput naming the
first problem found.
"""
import numpy as np


class InvalidInput(ValueError):
    pass


def decode_inputs(block_tables, context_lens, B: int, NB: int, max_context_len=None):
    """Block tables [S, MB] and context lengths [S] for decode (or prefill):
    0 <= L <= MB * B; the first ceil(L / B) entries of a row are physical
    blocks in [0, NB), distinct within the row (sequences may share a block,
    one sequence never holds it twice); max_context_len bounds every L."""
    tables = np.asarray(block_tables)
    lens = np.asarray(context_lens)
    if tables.ndim != 2:
        raise InvalidInput(f"block_tables must be [S, MB], got {tables.shape}")
    S, MB = tables.shape
    if lens.shape != (S,):
        raise InvalidInput(f"context_lens must be [{S}], got {lens.shape}")
    if S == 0:
        return
    if (lens < 0).any() or (lens > MB * B).any():
        s = int(np.argmax((lens < 0) | (lens > MB * B)))
        raise InvalidInput(f"sequence {s}: L = {int(lens[s])} outside [0, MB * B = {MB * B}]")
    if max_context_len is not None and int(lens.max()) > max_context_len:
        raise InvalidInput(f"max_context_len {max_context_len} below the longest L {int(lens.max())}")
    nblk = (lens.astype(np.int64) + B - 1) // B
    used = np.arange(MB)[None, :] < nblk[:, None]
    bad = used & ((tables < 0) | (tables >= NB))
    if bad.any():
        s, j = map(int, np.argwhere(bad)[0])
        raise InvalidInput(f"sequence {s}: table entry {j} = {int(tables[s, j])} outside [0, {NB})")
    for s in range(S):
        row = tables[s, :nblk[s]]
        if len(np.unique(row)) != len(row):
            raise InvalidInput(f"sequence {s}: a physical block appears twice in its table")


def write_batch(slot_mapping, B: int, NB: int):
    """Slots of one pa_write_kv call: negative means skip; the others lie in
    [0, NB * B) and no two tokens write the same slot."""
    slots = np.asarray(slot_mapping).astype(np.int64)
    live = slots[slots >= 0]
    if (live >= NB * B).any():
        raise InvalidInput(f"slot {int(live[live >= NB * B][0])} outside [0, {NB * B})")
    if len(np.unique(live)) != len(live):
        raise InvalidInput("two tokens of one call write the same slot")


def copy_pairs(block_mapping, NB_src: int, NB_dst: int = None, same_pool: bool = True):
    """(src, dst) pairs of one pa_copy_blocks / pa_swap_blocks call: ids in
    range; no block is written twice; within one pool no block is both a
    source and a destination (the pairs run in parallel)."""
    pairs = np.asarray(block_mapping).reshape(-1, 2).astype(np.int64)
    NB_dst = NB_src if NB_dst is None else NB_dst
    src, dst = pairs[:, 0], pairs[:, 1]
    if ((src < 0) | (src >= NB_src)).any():
        raise InvalidInput(f"source block outside [0, {NB_src})")
    if ((dst < 0) | (dst >= NB_dst)).any():
        raise InvalidInput(f"destination block outside [0, {NB_dst})")
    if len(np.unique(dst)) != len(dst):
        raise InvalidInput("a destination block is written twice")
    if same_pool and np.intersect1d(src, dst).size:
        raise InvalidInput("a block is both copied from and copied to in one call")


def prefill_inputs(block_tables, context_lens, query_start, T: int, B: int, NB: int,
                   max_query_len: int):
    """Tables and lengths as for decode, plus query_start [S + 1]: monotone in
    [0, T], each sequence's new tokens n = qs[s+1] - qs[s] at most its L (the
    new tokens are the last n of L) and at most max_query_len."""
    decode_inputs(block_tables, context_lens, B, NB)
    lens = np.asarray(context_lens).astype(np.int64)
    qs = np.asarray(query_start).astype(np.int64)
    if qs.shape != (len(lens) + 1,):
        raise InvalidInput(f"query_start must be [{len(lens) + 1}], got {qs.shape}")
    if (qs < 0).any() or (qs > T).any():
        raise InvalidInput(f"query_start outside [0, T = {T}]")
    n = np.diff(qs)
    if (n < 0).any():
        raise InvalidInput(f"query_start decreases at sequence {int(np.argmax(n < 0))}")
    if (n > lens).any():
        s = int(np.argmax(n > lens))
        raise InvalidInput(f"sequence {s}: {int(n[s])} new tokens but only L = {int(lens[s])}")
    if len(n) and int(n.max()) > max_query_len:
        raise InvalidInput(f"max_query_len {max_query_len} below {int(n.max())} new tokens")
