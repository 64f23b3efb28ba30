"""Pins of the prefix-caching block manager oracle (oracle/prefix_cache.py):
published FNV-1a test vectors, the worked example's FIFO order, closed forms
of sharing and eviction, and invariants over random request streams checked
against a simulated pool of token contents."""

import numpy as np
import pytest

from oracle import prefix_cache as pc
from tests import oracle_pins as pins


def test_fnv1a64_published_vectors():
    # test vectors of the FNV-1a 64-bit hash from its published definition
    assert pc.fnv1a64(b"") == 0xCBF29CE484222325
    assert pc.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert pc.fnv1a64(b"foobar") == 0x85944171F73967E8
    # continuing a hash equals hashing the concatenation
    assert pc.fnv1a64(b"bar", pc.fnv1a64(b"foo")) == pc.fnv1a64(b"foobar")
    assert pc.token_bytes([1, -1]) == b"\x01\x00\x00\x00\xff\xff\xff\xff"


def test_worked_example_fifo_order():
    g = pins.load_golden("worked_example.json")
    m = pc.PrefixCache(g["pool_blocks"], g["block_size"], caching=False, free=g["free_blocks"])
    sid, cached = m.add(list(range(g["num_keys"])))
    assert m.table(sid) == g["expected"]["block_table"] and cached == 0


class Checked:
    """Wraps the manager and a simulated pool of token contents; every write
    goes to a block with exactly one user and every sequence must read back
    its own tokens through its table."""

    def __init__(self, m: pc.PrefixCache, NB: int):
        self.m = m
        self.NB = NB
        self.pool = {}           # block -> list of bs entries (None = unwritten)
        self.tokens = {}         # seq -> tokens

    def _write(self, block, off, token):
        assert self.m.refs.get(block, 0) == 1, f"write into block {block} with {self.m.refs.get(block)} users"
        self.pool.setdefault(block, [None] * self.m.bs)[off] = token

    def add(self, toks):
        sid, cached = self.m.add(toks)
        bs = self.m.bs
        table = self.m.table(sid)
        assert cached % bs == 0 and cached <= len(toks)
        for p in range(cached):          # cached tokens are already in place
            assert self.pool[table[p // bs]][p % bs] == toks[p], "cached block holds other tokens"
        for p in range(cached, len(toks)):
            self._write(table[p // bs], p % bs, toks[p])
        self.tokens[sid] = list(toks)
        self.check()
        return sid, cached

    def append(self, sid, tok):
        slot, copy = self.m.append(sid, tok)
        if copy is not None:
            src, dst = copy
            self.pool[dst] = list(self.pool[src])
        self._write(slot // self.m.bs, slot % self.m.bs, tok)
        self.tokens[sid].append(tok)
        self.check()
        return slot, copy

    def fork(self, sid):
        nid = self.m.fork(sid)
        self.tokens[nid] = list(self.tokens[sid])
        self.check()
        return nid

    def free(self, sid):
        self.m.free_seq(sid)
        del self.tokens[sid]
        self.check()

    def check(self):
        m, bs = self.m, self.m.bs
        users = {}
        for sid, toks in self.tokens.items():
            table = m.table(sid)
            assert len(table) == -(-len(toks) // bs)
            for p, t in enumerate(toks):
                assert self.pool[table[p // bs]][p % bs] == t, (sid, p)
            for b in table:
                users[b] = users.get(b, 0) + 1
        assert users == m.refs
        free, evict = set(m.free), set(m.evictable)
        assert len(free) == len(m.free) and len(evict) == len(m.evictable)
        assert not (free & evict) and not (free & set(users)) and not (evict & set(users))
        assert len(free) + len(evict) + len(users) == self.NB
        assert set(m.key) == set(m.owner.values()) and evict <= set(m.key)
        for b in m.key:                 # a keyed block is full and holds its tokens
            assert self.pool[b] == m.meta[b][1]


def test_identical_prompts_share_every_full_block():
    m = Checked(pc.PrefixCache(64, 16), 64)
    prompt = list(range(1000, 1000 + 16 * 5 + 7))
    a, ca = m.add(prompt)
    b, cb = m.add(prompt)
    assert (ca, cb) == (0, 80)
    assert m.m.table(a)[:5] == m.m.table(b)[:5] and m.m.table(a)[5] != m.m.table(b)[5]
    c, cc = m.add(prompt[:40] + [7] * 30)            # shares two full blocks, then differs
    assert cc == 32 and m.m.table(c)[:2] == m.m.table(a)[:2]
    d, cd = m.add([5] * 48)                           # disjoint: shares nothing
    assert cd == 0 and not set(m.m.table(d)) & set(m.m.table(a))
    # same second block after a different first one: nothing is shared (a
    # block's K/V depend on every token before it, so the key covers them)
    f, cf = m.add([3] * 16 + prompt[16:32] + [4])
    assert cf == 0 and m.m.table(f)[1] != m.m.table(a)[1]
    for s in (a, b, c, d, f):
        m.free(s)
    # the keyed blocks stay cached: the same prompt hits them again
    e, ce = m.add(prompt)
    assert ce == 80


def test_eviction_takes_the_longest_released_cached_block():
    m = Checked(pc.PrefixCache(6, 4), 6)
    a, _ = m.add([1, 2, 3, 4, 5, 6, 7, 8])           # 2 keyed blocks
    b, _ = m.add([9, 9, 9, 9])                        # 1 keyed block
    ta, tb = m.m.table(a), m.m.table(b)
    m.free(a)                                          # released last block first
    m.free(b)
    assert m.m.evictable == [ta[1], ta[0], tb[0]] and len(m.m.free) == 3
    c, cc = m.add([0] * 16)                            # 4 blocks: 3 free + the oldest cached one
    assert cc == 0 and ta[1] in m.m.table(c)
    # 3 keys, one lost with the evicted block, 4 new ones (chained: all distinct)
    assert m.m.cached_blocks() == 6
    assert m.m.evictable == [ta[0], tb[0]]
    d, cd = m.add([1, 2, 3, 4])                        # a's first block is still cached
    assert cd == 4 and m.m.table(d) == [ta[0]]


def test_out_of_blocks_changes_nothing():
    m = pc.PrefixCache(4, 4)
    a, _ = m.add(list(range(12)))
    before = (list(m.free), list(m.evictable), dict(m.refs), dict(m.owner))
    with pytest.raises(pc.OutOfBlocks):
        m.add(list(range(100, 108)))
    assert (list(m.free), list(m.evictable), dict(m.refs), dict(m.owner)) == before
    b = m.fork(a)
    m.append(b, 5)                                     # position 12: a new block, the last one
    with pytest.raises(pc.OutOfBlocks):
        m.append(a, 6)
    assert m.length(a) == 12


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("caching", [True, False])
def test_random_streams_keep_every_invariant(seed, caching):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([1, 2, 4, 16]))
    NB = int(rng.integers(20, 80))
    m = Checked(pc.PrefixCache(NB, bs, caching=caching, free=list(rng.permutation(NB))), NB)
    systems = [list(rng.integers(0, 50, size=int(rng.integers(1, 5 * bs)))) for _ in range(3)]
    live = []
    for _ in range(150):
        op = rng.integers(0, 10)
        try:
            if op < 3 or not live:
                sys_p = systems[int(rng.integers(3))]
                tail = list(rng.integers(0, 50, size=int(rng.integers(0, 2 * bs + 2))))
                toks = sys_p + tail if sys_p + tail else [1]
                live.append(m.add(toks)[0])
            elif op < 7:
                m.append(live[int(rng.integers(len(live)))], int(rng.integers(0, 50)))
            elif op < 8:
                live.append(m.fork(live[int(rng.integers(len(live)))]))
            else:
                s = live.pop(int(rng.integers(len(live))))
                m.free(s)
        except pc.OutOfBlocks:
            if live:
                m.free(live.pop(0))


# ---------------------------------------------------------------- mutants

class UnchainedKeys(pc.PrefixCache):
    """Keys from each block's own tokens only."""

    def _keys(self, tokens):
        return [(pc.fnv1a64(pc.token_bytes(tokens[j * self.bs:(j + 1) * self.bs])), pc.FNV_OFFSET)
                for j in range(len(tokens) // self.bs)]


class NewestEvictedFirst(pc.PrefixCache):
    def _take(self):
        if not self.free and self.evictable:
            self.evictable.insert(0, self.evictable.pop())
        return super()._take()


class NoCopyOnWrite(pc.PrefixCache):
    def append(self, sid, token):
        s = self.seqs[sid]
        p = len(s["tokens"])
        if p % self.bs:
            s["tokens"].append(int(token))
            return s["table"][p // self.bs] * self.bs + p % self.bs, None
        return super().append(sid, token)


class FirstBlockReleasedFirst(pc.PrefixCache):
    def free_seq(self, sid):
        s = self.seqs.pop(sid)
        for b in s["table"]:
            self._release(b)


@pytest.mark.parametrize("cls", [UnchainedKeys, NewestEvictedFirst, NoCopyOnWrite, FirstBlockReleasedFirst])
def test_mutants_are_caught(cls, monkeypatch):
    monkeypatch.setattr(pc, "PrefixCache", cls)
    failed = False
    for t in (test_identical_prompts_share_every_full_block,
              test_eviction_takes_the_longest_released_cached_block):
        try:
            t()
        except AssertionError:
            failed = True
    if not failed:
        for seed in range(12):
            try:
                test_random_streams_keep_every_invariant(seed, True)
            except AssertionError:
                failed = True
                break
    assert failed, cls.__name__
