"""Invariants of the oracle's block bookkeeping over random operation sequences.

Pins (P1 "Sayfalama Nasıl Çalışır", "Diziler Arasında Blokları Paylaşma";
P3 article A): a sequence always reads back exactly its own tokens through its
table; a block is only written while it has one user; reference counts equal
the number of tables that hold each block; freed blocks return to the pool;
a new block is taken only when the last one is full.
"""

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import blocks, paged

BS = 4
NB = 48

ops = st.lists(st.tuples(st.sampled_from(["new", "fork", "append", "append", "append", "free"]),
                         st.integers(0, 1000), st.integers(0, 9)), min_size=1, max_size=60)


def check_invariants(pool, seqs, content):
    counts = {}
    for s in seqs:
        for b in s["table"]:
            counts[b] = counts.get(b, 0) + 1
        got = paged.gather(content, np.array(s["table"]), s["len"], BS)
        assert list(got) == s["tokens"], "a sequence must read back its own tokens"
        assert len(s["table"]) == -(-s["len"] // BS), "blocks only when the last one is full"
    assert counts == pool.refs
    assert not set(pool.free) & set(pool.refs)
    assert len(pool.free) + len(pool.refs) == NB


@settings(max_examples=150, deadline=None)
@given(ops=ops, seed=st.integers(0, 2 ** 31 - 1))
def test_block_bookkeeping_invariants(ops, seed):
    rng = np.random.default_rng(seed)
    pool = blocks.BlockPool(free=[int(b) for b in rng.permutation(NB)])
    content = np.full((NB, BS), -1, dtype=np.int64)
    seqs, next_tok = [], 0
    for op, a, n in ops:
        try:
            if op == "new" or not seqs:
                L = n + 1
                table = blocks.allocate_sequence(pool, L, BS)
                toks = list(range(next_tok, next_tok + L))
                next_tok += L
                for pos, t in enumerate(toks):
                    slot = table[pos // BS] * BS + pos % BS
                    content[slot // BS, slot % BS] = t
                seqs.append(dict(table=table, len=L, tokens=toks))
            elif op == "fork":
                s = seqs[a % len(seqs)]
                seqs.append(dict(table=blocks.fork(pool, s["table"]), len=s["len"], tokens=list(s["tokens"])))
            elif op == "append":
                s = seqs[a % len(seqs)]
                slot, cow = blocks.append_slot(pool, s["table"], s["len"], BS)
                if cow is not None:
                    content = paged.copy_blocks(content, np.array([cow]))
                blk = slot // BS
                assert pool.refs[blk] == 1, "write into a block that others still use"
                content[blk, slot % BS] = next_tok
                s["tokens"].append(next_tok)
                s["len"] += 1
                next_tok += 1
            elif op == "free":
                s = seqs.pop(a % len(seqs))
                for b in s["table"]:
                    pool.release(b)
        except blocks.OutOfBlocks:
            # allocation may fail part-way through a new sequence; undo it
            if op == "new":
                held = [b for b in pool.refs if not any(b in s["table"] for s in seqs)]
                for b in held:
                    pool.release(b)
            continue
        check_invariants(pool, seqs, content)


def test_shared_stem_copy_order():
    """Three samples sharing a partial last block: the first two writers copy
    it, the last one writes in place (the count drops 3 -> 2 -> 1)."""
    pool = blocks.BlockPool(free=list(range(20)))
    base = blocks.allocate_sequence(pool, 6, BS)           # blocks [0, 1], last one partial
    tables = [base] + [blocks.fork(pool, base) for _ in range(2)]
    assert pool.refs[1] == 3
    cows = []
    for t in tables:
        _, cow = blocks.append_slot(pool, t, 6, BS)
        cows.append(cow)
    assert cows == [(1, 2), (1, 3), None]
    assert [t[1] for t in tables] == [2, 3, 1]
    assert pool.refs == {0: 3, 1: 1, 2: 1, 3: 1}
