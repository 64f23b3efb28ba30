"""Host-side block bookkeeping the pages describe (test infrastructure only).

* Free list, FIFO: P1's code sketch ("Sayfalama Nasıl Çalışır") hands out
  blocks by popping the front of a list of scattered free block ids.
* On-demand allocation: a sequence takes a new block only when its last block
  is full (P1 "Sayfalama Nasıl Çalışır"; P3 article A, on-demand allocation).
* Sharing with reference counts and copy-on-write: several sequences may point
  at one physical block; each block carries a count of its users, and a
  sequence about to write into a block that others still use first gets a
  private copy (P1 "Diziler Arasında Blokları Paylaşma"; P3 article A,
  shared prefix support).
* Freed blocks return to the pool at once (P1 "İlgili Teknikler", continuous
  batching).

Pinned by the worked example (the sketch's free list [41, 7, 19, 2, 33] gives
the table [41, 7, 19]) and by invariants checked over random layouts: after a
planned step every sequence still sees exactly its own tokens, no block with
more than one user is written, and counts equal the number of tables that
reference each block.
"""

from __future__ import annotations

from dataclasses import dataclass, field


class OutOfBlocks(RuntimeError):
    """The free list is empty."""


@dataclass
class BlockPool:
    """FIFO free list plus a reference count per block in use."""

    free: list
    refs: dict = field(default_factory=dict)

    def allocate(self) -> int:
        if not self.free:
            raise OutOfBlocks("no free block left")
        b = int(self.free.pop(0))
        self.refs[b] = 1
        return b

    def share(self, b: int) -> None:
        self.refs[b] += 1

    def release(self, b: int) -> None:
        self.refs[b] -= 1
        if self.refs[b] == 0:
            del self.refs[b]
            self.free.append(b)


def allocate_sequence(pool: BlockPool, length: int, block_size: int) -> list:
    """Block table for a new sequence of ``length`` tokens: ceil(L / bs) blocks
    popped from the front of the free list, in logical order."""
    n = -(-int(length) // int(block_size))
    return [pool.allocate() for _ in range(n)]


def fork(pool: BlockPool, table: list) -> list:
    """A new sequence sharing every block of ``table`` (refcounts + 1)."""
    for b in table:
        pool.share(b)
    return list(table)


def append_slot(pool: BlockPool, table: list, length: int, block_size: int):
    """Plan the write of token number ``length`` (0-based position) of a sequence.

    Returns ``(slot, cow)`` and updates ``table`` and the pool in place:

    * position % bs == 0: the last block is full (or there is none), so a new
      block is taken from the free list;
    * else, if the last block has other users: take a new block, record the
      copy ``(old, new)``, drop one reference to the old block and point the
      table at the new one;
    * else write in place.

    ``cow`` is ``None`` or the ``(src, dst)`` pair.
    """
    pos = int(length)
    cow = None
    if pos % block_size == 0:
        if pos // block_size != len(table):
            raise ValueError("table length does not match the sequence length")
        table.append(pool.allocate())
    else:
        last = table[pos // block_size]
        if pool.refs[last] > 1:
            new = pool.allocate()
            pool.refs[last] -= 1
            table[pos // block_size] = new
            cow = (last, new)
    slot = table[pos // block_size] * block_size + pos % block_size
    return slot, cow
