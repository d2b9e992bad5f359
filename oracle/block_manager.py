"""Host block manager with reference counts and copy-on-write
(oracle fixture; test infrastructure only).

[L] = "Paged Attention: OS-Inspired Memory Management for KV Caches",
sections "How PagedAttention works", "Memory sharing across requests" and
"Practice: try it yourself".

Behaviour:
  * a free list of physical ids, handed out from the front;
  * every block has a reference count (sequences using it) and a fill count
    (slots already written);
  * appending a token to a sequence: if it has no block or its last block is
    full, a fresh block is taken; otherwise, if the last block is shared
    (count > 1), the sequence gets a fresh block holding a copy of the slots
    written so far, the old block's count drops by one and the table entry is
    repointed; the token then takes the next slot of the last block;
  * fork: a new sequence shares every block of its parent (counts + 1);
  * release: each block's count drops by one and blocks that reach zero go
    back to the free list.
Every copy is recorded as a (src, dst) pair: the device-side copy that the
library's block-copy call performs.
"""
from __future__ import annotations


class PoolExhausted(RuntimeError):
    """No free block is left; a server must queue or preempt
    ([L], "Worked example, step by step", last paragraph)."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        self.block_size = int(block_size)
        self.free = list(range(int(num_blocks)))
        self.refs: dict[int, int] = {}
        self.fill: dict[int, int] = {}
        self.copies: list[tuple[int, int]] = []

    def _take(self) -> int:
        if not self.free:
            raise PoolExhausted("no free block")
        b = self.free.pop(0)
        self.refs[b] = 1
        self.fill[b] = 0
        return b

    def append_token(self, table: list) -> int:
        """Place one new token; returns its pool-wide slot (block * B + offset)."""
        last = table[-1] if table else None
        if last is None or self.fill[last] == self.block_size:
            table.append(self._take())
        elif self.refs[last] > 1:
            fresh = self._take()
            self.fill[fresh] = self.fill[last]
            self.refs[last] -= 1
            self.copies.append((last, fresh))
            table[-1] = fresh
        blk = table[-1]
        off = self.fill[blk]
        self.fill[blk] = off + 1
        return blk * self.block_size + off

    def fork(self, table: list) -> list:
        for b in table:
            self.refs[b] += 1
        return list(table)

    def release(self, table: list) -> list:
        """Drop one reference per block; returns the ids that became free."""
        freed = []
        for b in table:
            self.refs[b] -= 1
            if self.refs[b] == 0:
                del self.refs[b]
                del self.fill[b]
                self.free.append(b)
                freed.append(b)
        table.clear()
        return freed

    def blocks_in_use(self) -> int:
        return len(self.refs)
