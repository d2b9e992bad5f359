"""Host block manager with reference counts and copy-on-write
(oracle fixture; test infrastructure only).

[L] = "Paged Attention: OS-Inspired Memory Management for KV Caches".
The rules, from the prose of its sections "How PagedAttention works" (the life
of one request) and "Memory sharing across requests":

  * a request's cache is a block table, physical ids in logical order, plus
    the number of tokens it holds; token t lives in logical block t // B at
    offset t % B;
  * prefill takes just enough blocks (ceil(L / B)), and each new token goes
    into the next slot of the last block; only when that slot lies past the
    last block is one more free block taken (allocation on demand);
  * a block keeps a count of the sequences that use it; forking a sequence
    (parallel sampling, beam search, a shared prompt) lets the new one use
    every block of the old one, adding one to each count;
  * before a token is written into a block whose count is above one, the
    writer gets a fresh block holding a copy of it (copy-on-write): its table
    points at the copy, the original's count drops by one, then the token is
    written; full blocks are never written again, so only a partly filled last
    block is ever copied;
  * when a request finishes, each of its blocks loses one count, and blocks
    whose count reaches zero return to the free list.

Free blocks are handed out from the front of the list and returned to its
back. Every copy is recorded as a (src, dst) pair: the device-side copy that
the library's block-copy call performs. The page's practice trace (printed
under "Practice: try it yourself") and its pause-and-think answers are the
golden data this manager is checked against.
"""
from __future__ import annotations

from collections import deque


class PoolExhausted(RuntimeError):
    """No free block is left; a server must queue or preempt
    ([L], "Worked example, step by step", last paragraph)."""


class Sequence:
    """One request's view of the cache: its block table and token count."""

    __slots__ = ("blocks", "length")

    def __init__(self, blocks=None, length: int = 0):
        self.blocks: list[int] = list(blocks or [])
        self.length = int(length)

    def __repr__(self) -> str:
        return f"Sequence(blocks={self.blocks}, length={self.length})"


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        self.B = int(block_size)
        self.count = [0] * int(num_blocks)       # sequences using each block; 0 = free
        self.free_list = deque(range(int(num_blocks)))
        self.copies: list[tuple[int, int]] = []

    # -- pool ---------------------------------------------------------------
    def _take_free_block(self) -> int:
        if not self.free_list:
            raise PoolExhausted("no free block")
        b = self.free_list.popleft()
        self.count[b] = 1
        return b

    def refcount(self, block: int) -> int:
        return self.count[block]

    def blocks_in_use(self) -> int:
        return sum(1 for c in self.count if c > 0)

    # -- sequences ----------------------------------------------------------
    def new_sequence(self) -> Sequence:
        return Sequence()

    def append(self, seq: Sequence) -> int:
        """Write one new token at position seq.length; returns its pool-wide
        slot (block * B + offset). On PoolExhausted nothing has changed."""
        j, off = divmod(seq.length, self.B)
        if j == len(seq.blocks):
            # the position lies past the last block: allocate on demand
            seq.blocks.append(self._take_free_block())
        elif self.count[seq.blocks[j]] > 1:
            # the block is shared: the writer gets its own copy first
            shared = seq.blocks[j]
            own = self._take_free_block()
            self.copies.append((shared, own))
            self.count[shared] -= 1
            seq.blocks[j] = own
        seq.length += 1
        return seq.blocks[j] * self.B + off

    def fork(self, seq: Sequence) -> Sequence:
        """A new sequence that shares every block (and token) of `seq`."""
        for b in seq.blocks:
            self.count[b] += 1
        return Sequence(seq.blocks, seq.length)

    def free(self, seq: Sequence) -> list:
        """The request is finished: drop its references; returns the blocks
        that became free, in the order they joined the free list."""
        freed = []
        for b in seq.blocks:
            self.count[b] -= 1
            if self.count[b] == 0:
                self.free_list.append(b)
                freed.append(b)
        seq.blocks = []
        seq.length = 0
        return freed
