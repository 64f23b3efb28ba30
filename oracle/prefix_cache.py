"""Host block manager with content-hashed prefix caching, restated plainly
(test infrastructure only).

What it follows:

* Blocks come from the front of a FIFO free list and go back to its end
  (P1 "Sayfalama Nasıl Çalışır": the code sketch pops free blocks from the
  front of a list of scattered ids).
* A sequence takes a new block only when its last one is full (same section;
  P3 article A, on-demand allocation).
* Sequences may point at the same blocks, each block counting its users; a
  sequence about to write into a block others still use gets a copy first
  (P1 "Diziler Arasında Blokları Paylaşma"; P3 article A).
* Hashing every block lets requests that start with the same tokens share
  their cached blocks (P1 "Diziler Arasında Blokları Paylaşma": prompt
  caching).  A finished sequence's blocks return at once (P1 "İlgili
  Teknikler", continuous batching).

The pages give no more than that; the readings below fix the rest, and the
native manager in the library follows the same readings.

* A full block's key is the 64-bit FNV-1a hash of every token from the
  start of the sequence through the end of that block, the token ids taken
  as 4-byte little-endian integers (FNV-1a: start from the offset basis
  0xcbf29ce484222325; per byte, xor it in, then multiply by the prime
  0x100000001b3 modulo 2^64).  A cached block also keeps its own tokens and
  its parent's key; a lookup hits only when all three match.  Only full
  blocks are keyed.
* Admitting a prompt reuses cached blocks for its leading full blocks, in
  order, and stops at the first block that misses.  The rest are new blocks;
  each new full block registers its key unless the key is already taken.
* A new block comes from the front of the free list; when the list is empty,
  the cached block with no users that was released longest ago is taken and
  loses its key.  With neither, the operation fails and changes nothing.
* Appending token t at position p: p % bs == 0 takes a new block; otherwise,
  if the last block has other users, a new block replaces it in this
  sequence's table (the copy (old, new) is reported and the old block loses
  one user).  When the append fills the block, the block registers its key
  (if it has none and the key is not taken).
* Freeing a sequence releases its blocks last block first; a block whose
  last user leaves goes to the back of the evictable list if it has a key,
  else to the back of the free list.

Every operation is pinned in tests/test_oracle_prefix_cache.py by invariants
(each sequence reads back exactly its own tokens through its table, reference
counts equal the tables' references, a block with several users is never
written, free and cached blocks are disjoint and account for the pool),
closed forms (identical prompts share every full block; disjoint prompts
share none; the worked example's FIFO order) and the published FNV-1a test
vectors.
"""

from __future__ import annotations

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """FNV-1a, 64 bits, continued from ``h``."""
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def token_bytes(tokens) -> bytes:
    """Token ids as 4-byte little-endian two's-complement integers."""
    return b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens)


class OutOfBlocks(RuntimeError):
    """Neither a free nor an evictable block is left."""


class PrefixCache:
    def __init__(self, num_blocks: int, block_size: int, caching: bool = True, free=None):
        self.bs = int(block_size)
        self.caching = bool(caching)
        self.free = list(range(num_blocks)) if free is None else [int(b) for b in free]
        self.evictable = []          # blocks with a key and no user, oldest release first
        self.refs = {}               # block -> users
        self.key = {}                # block -> key
        self.owner = {}              # key -> block
        self.meta = {}               # block -> (parent key, tokens of the block)
        self.seqs = {}               # seq id -> {"tokens": [...], "table": [...]}
        self.next_id = 0

    # ---------------------------------------------------------------- helpers

    def _keys(self, tokens):
        """Key of every full block of ``tokens``, with its parent's key."""
        out, h = [], FNV_OFFSET
        for j in range(len(tokens) // self.bs):
            parent = h
            h = fnv1a64(token_bytes(tokens[j * self.bs:(j + 1) * self.bs]), h)
            out.append((h, parent))
        return out

    def _lookup(self, k, parent, toks):
        b = self.owner.get(k)
        if b is None:
            return None
        if self.meta[b] != (parent, list(toks)):
            return None
        return b

    def _available(self):
        return len(self.free) + len(self.evictable)

    def _take(self):
        if self.free:
            b = self.free.pop(0)
        elif self.evictable:
            b = self.evictable.pop(0)
            k = self.key.pop(b)
            del self.owner[k]
            del self.meta[b]
        else:
            raise OutOfBlocks("no free or evictable block")
        self.refs[b] = 1
        return b

    def _register(self, b, k, parent, toks):
        if not self.caching or b in self.key or k in self.owner:
            return
        self.key[b] = k
        self.owner[k] = b
        self.meta[b] = (parent, list(toks))

    def _release(self, b):
        self.refs[b] -= 1
        if self.refs[b] == 0:
            del self.refs[b]
            if b in self.key:
                self.evictable.append(b)
            else:
                self.free.append(b)

    # ---------------------------------------------------------------- operations

    def add(self, tokens):
        """Admit a sequence with ``tokens``; returns (seq id, cached tokens)."""
        tokens = [int(t) for t in tokens]
        keys = self._keys(tokens) if self.caching else []
        hits = []
        for j, (k, parent) in enumerate(keys):
            b = self._lookup(k, parent, tokens[j * self.bs:(j + 1) * self.bs])
            if b is None:
                break
            hits.append(b)
        nblocks = -(-len(tokens) // self.bs)
        revived = sum(1 for b in hits if b in self.evictable)
        if nblocks - len(hits) > self._available() - revived:
            raise OutOfBlocks("not enough blocks for the prompt")
        table = []
        for b in hits:
            if b in self.evictable:
                self.evictable.remove(b)
                self.refs[b] = 1
            else:
                self.refs[b] += 1
            table.append(b)
        for j in range(len(hits), nblocks):
            b = self._take()
            table.append(b)
            if j < len(keys):
                k, parent = keys[j]
                self._register(b, k, parent, tokens[j * self.bs:(j + 1) * self.bs])
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = {"tokens": tokens, "table": table}
        return sid, len(hits) * self.bs

    def append(self, sid, token):
        """Append one token; returns (slot, copy pair or None)."""
        s = self.seqs[sid]
        p = len(s["tokens"])
        table = s["table"]
        copy = None
        if p % self.bs == 0:
            if self._available() < 1:
                raise OutOfBlocks("no block for the new token")
            table.append(self._take())
        else:
            last = table[p // self.bs]
            if self.refs[last] > 1:
                if self._available() < 1:
                    raise OutOfBlocks("no block for the copy")
                new = self._take()
                self.refs[last] -= 1
                table[p // self.bs] = new
                copy = (last, new)
        s["tokens"].append(int(token))
        slot = table[p // self.bs] * self.bs + p % self.bs
        if (p + 1) % self.bs == 0 and self.caching:
            j = p // self.bs
            k, parent = self._keys(s["tokens"])[j]
            self._register(table[j], k, parent, s["tokens"][j * self.bs:(j + 1) * self.bs])
        return slot, copy

    def fork(self, sid):
        """A new sequence sharing every block of ``sid``."""
        s = self.seqs[sid]
        for b in s["table"]:
            self.refs[b] += 1
        nid = self.next_id
        self.next_id += 1
        self.seqs[nid] = {"tokens": list(s["tokens"]), "table": list(s["table"])}
        return nid

    def free_seq(self, sid):
        s = self.seqs.pop(sid)
        for b in reversed(s["table"]):
            self._release(b)

    def table(self, sid):
        return list(self.seqs[sid]["table"])

    def length(self, sid):
        return len(self.seqs[sid]["tokens"])

    def free_blocks(self):
        return self._available()

    def cached_blocks(self):
        return len(self.key)
