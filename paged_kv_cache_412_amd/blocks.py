"""Host block manager: plans one decode step's cache writes.

P1 = Ultralytics glossary page "PagedAttention"; P3 = gyaansetu.com page on KV
memory and PagedAttention.

* A sequence takes a new block only when its last block is full, from the
  front of the free list (P1 "Sayfalama Nasıl Çalışır", code sketch; P3
  article A, on-demand allocation).
* Blocks carry reference counts; a sequence that is about to write into a
  block other sequences still use gets a fresh block and a copy first
  (copy-on-write, P1 "Diziler Arasında Blokları Paylaşma"; P3 article A,
  shared prefix support).

The manager only decides which block each table points at and which blocks
must be copied; the slots themselves are computed on the GPU
(``pa_slot_mapping``) and the copies run there (``pa_copy_blocks``).
"""

from __future__ import annotations

from collections import deque

import numpy as np


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    """Free list (FIFO) plus per-block reference counts over a pool of blocks."""

    def __init__(self, num_blocks: int, block_size: int, free=None, refs=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.free = deque(int(b) for b in (range(num_blocks) if free is None else free))
        self.refcount = np.zeros(self.num_blocks, dtype=np.int64)
        for blk, n in (refs or {}).items():
            self.refcount[int(blk)] = int(n)

    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks("the block pool is exhausted")
        blk = self.free.popleft()
        self.refcount[blk] = 1
        return blk

    def release(self, table) -> None:
        """A finished sequence hands its blocks back (P1 "İlgili Teknikler",
        continuous batching)."""
        for blk in table:
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                self.free.append(int(blk))

    def plan_step(self, tables: list, cached_lens) -> tuple:
        """Make room for one new token per sequence.

        ``tables[i]`` lists the blocks of sequence i, which holds
        ``cached_lens[i]`` tokens; the new token goes to position
        ``cached_lens[i]`` (a negative entry means the sequence gets no new
        token).  Sequences are handled in order.  Returns
        ``(new_tables, copies)``: updated tables and the list of
        ``(src, dst)`` block copies to run before the cache write.
        """
        bs = self.block_size
        out, copies = [], []
        for row, n in zip(tables, cached_lens):
            row = list(row)
            n = int(n)
            if n < 0:
                out.append(row)
                continue
            j = n // bs
            if n % bs == 0:                       # last block full (or none yet)
                if len(row) != j:
                    raise ValueError("table does not match the cached length")
                row.append(self._take())
            elif self.refcount[row[j]] > 1:       # shared partial block: copy on write
                old = row[j]
                new = self._take()
                self.refcount[old] -= 1
                row[j] = new
                copies.append((old, new))
            out.append(row)
        return out, copies
