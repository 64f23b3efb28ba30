"""Checks that pin the oracle to facts outside itself.

Each ``check_*`` takes the oracle function(s) it exercises as arguments and
raises ``AssertionError`` when they disagree with the pages, a closed form, a
library routine or brute force.  ``tests/test_oracle_*.py`` runs them on the
oracle; ``tests/test_oracle_mutants.py`` runs them on deliberately broken
copies of oracle functions and requires each copy to be caught.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


# --------------------------------------------------------------------------
# P1 "Sayfalama Nasıl Çalışır": the worked example (code sketch + its output)
# --------------------------------------------------------------------------

def check_worked_example(BlockPool, allocate_sequence, slot_mapping, write_cache, gather,
                         paged_unused_slots, reserved_unused_slots, seed=0):
    g = load_golden("worked_example.json")
    ex = g["expected"]
    bs, D, NB = g["block_size"], g["head_dim"], g["pool_blocks"]
    pool = BlockPool(free=list(g["free_blocks"]))
    table = allocate_sequence(pool, g["num_keys"], bs)
    assert len(table) == ex["blocks_needed"], table
    assert list(table) == ex["block_table"], table
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((g["num_keys"], 1, D)).astype(np.float32)
    key_pool = np.zeros((NB, bs, 1, D), dtype=np.float32)
    tables = np.array([table], dtype=np.int32)
    for pos in range(g["num_keys"]):
        slot = slot_mapping(tables, np.array([pos]), bs)
        key_pool = write_cache(key_pool, keys[pos:pos + 1], slot, bs)
    back = gather(key_pool, tables[0], g["num_keys"], bs)
    intact = back.shape == keys.shape and np.array_equal(back.view(np.uint32), keys.view(np.uint32))
    assert intact == ex["keys_intact"]
    # nothing outside the three blocks was touched
    others = np.setdiff1d(np.arange(NB), table)
    assert not key_pool[others].any()
    assert paged_unused_slots(g["num_keys"], bs) == ex["unused_slots_paged"]
    assert reserved_unused_slots(g["num_keys"], g["reservation"]) == ex["unused_slots_reserved"]


# --------------------------------------------------------------------------
# attention: library special case, brute force and closed forms
# --------------------------------------------------------------------------

def random_paged(rng, B, Hq, Hkv, D, bs, lens, NB=None, poison=True):
    """Random pools + scattered tables for oracle checks (float64 values)."""
    need = sum(-(-int(L) // bs) for L in lens)
    NB = NB or need + 3
    perm = rng.permutation(NB)
    tables = np.full((B, max(1, max(-(-int(L) // bs) for L in lens)) + 1), -1, dtype=np.int64)
    k = 0
    for b, L in enumerate(lens):
        n = -(-int(L) // bs)
        tables[b, :n] = perm[k:k + n]
        k += n
    kp = rng.standard_normal((NB, bs, Hkv, D))
    vp = rng.standard_normal((NB, bs, Hkv, D))
    if poison:
        used = np.zeros(NB, bool)
        for b, L in enumerate(lens):
            n = -(-int(L) // bs)
            used[tables[b, :n]] = True
            if L % bs:
                kp[tables[b, n - 1], L % bs:] = np.nan
                vp[tables[b, n - 1], L % bs:] = np.nan
        kp[~used] = np.nan
        vp[~used] = np.nan
    q = rng.standard_normal((B, Hq, D))
    return q, kp, vp, tables, np.asarray(lens, dtype=np.int64)


def contiguous(pool, tables, lens, bs):
    """Per-sequence contiguous [L, Hkv, D] by explicit slot indexing (not the oracle's gather)."""
    out = []
    for b, L in enumerate(lens):
        rows = [pool[tables[b, t // bs], t % bs] for t in range(int(L))]
        out.append(np.stack(rows) if rows else np.zeros((0,) + pool.shape[2:]))
    return out


def check_decode_vs_sdpa(decode, seed=1, B=3, Hq=8, Hkv=2, D=16, bs=4, lens=(1, 7, 13)):
    """fp64 torch scaled_dot_product_attention on contiguous K/V, with KV heads
    repeated for consecutive query heads (h -> h // G)."""
    rng = np.random.default_rng(seed)
    q, kp, vp, tables, lens = random_paged(rng, B, Hq, Hkv, D, bs, lens)
    scale = 0.37
    out = decode(q, kp, vp, tables, lens, bs, scale)
    G = Hq // Hkv
    ks, vs = contiguous(kp, tables, lens, bs), contiguous(vp, tables, lens, bs)
    for b in range(B):
        K = torch.from_numpy(ks[b]).permute(1, 0, 2).repeat_interleave(G, dim=0)   # [Hq, L, D]
        V = torch.from_numpy(vs[b]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        Q = torch.from_numpy(q[b]).unsqueeze(1)                                      # [Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[:, 0, :].numpy()
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def check_decode_vs_bruteforce(decode, seed=2, B=2, Hq=4, Hkv=2, D=5, bs=3, lens=(5, 8)):
    """Pure-Python loops with math.exp over explicit slot indices."""
    rng = np.random.default_rng(seed)
    q, kp, vp, tables, lens = random_paged(rng, B, Hq, Hkv, D, bs, lens)
    scale = 0.61
    out = decode(q, kp, vp, tables, lens, bs, scale)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // G
            scores = []
            for t in range(int(lens[b])):
                blk, off = int(tables[b, t // bs]), t % bs
                scores.append(scale * sum(float(q[b, h, d]) * float(kp[blk, off, g, d]) for d in range(D)))
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = sum(w)
            for d in range(D):
                acc = 0.0
                for t in range(int(lens[b])):
                    blk, off = int(tables[b, t // bs]), t % bs
                    acc += w[t] * float(vp[blk, off, g, d])
                assert abs(out[b, h, d] - acc / tot) <= 1e-12 * max(1.0, abs(acc / tot)), (b, h, d)


def check_closed_forms(decode, seed=3):
    rng = np.random.default_rng(seed)
    bs, D = 4, 8
    # L = 1: a single weight of exactly 1, so out equals v_0 bit for bit
    q, kp, vp, tables, lens = random_paged(rng, 2, 4, 4, D, bs, (1, 1))
    out = decode(q, kp, vp, tables, lens, bs, 0.5)
    for b in range(2):
        assert np.array_equal(out[b], vp[tables[b, 0], 0]), "L=1 must return v_0 exactly"
    # q = 0: uniform weights, out = mean of the L value rows
    q, kp, vp, tables, lens = random_paged(rng, 1, 2, 2, D, bs, (11,))
    q[:] = 0.0
    out = decode(q, kp, vp, tables, lens, bs, 0.5)
    rows = np.stack([vp[tables[0, t // bs], t % bs] for t in range(11)])
    np.testing.assert_allclose(out[0], rows.mean(axis=0), rtol=0, atol=1e-14)
    # planted dominant key: out -> that key's value row
    q, kp, vp, tables, lens = random_paged(rng, 1, 1, 1, D, bs, (9,))
    t0 = 6
    kp[tables[0, t0 // bs], t0 % bs, 0] = 60.0 * q[0, 0] / np.linalg.norm(q[0, 0])
    out = decode(q, kp, vp, tables, lens, bs, 1.0)
    np.testing.assert_allclose(out[0, 0], vp[tables[0, t0 // bs], t0 % bs, 0], rtol=0, atol=1e-12)
    # L = 0: zeros
    q, kp, vp, tables, lens = random_paged(rng, 2, 2, 2, D, bs, (0, 3))
    out = decode(q, kp, vp, tables, lens, bs, 0.5)
    assert np.array_equal(out[0], np.zeros_like(out[0]))


def check_placement_invariance(decode, seed=4):
    """Any permutation of physical blocks, applied to pool and tables, leaves
    the output bit-identical (P1: blocks may sit anywhere in memory)."""
    rng = np.random.default_rng(seed)
    bs = 4
    q, kp, vp, tables, lens = random_paged(rng, 3, 4, 2, 8, bs, (9, 16, 3))
    out = decode(q, kp, vp, tables, lens, bs, 0.3)
    NB = kp.shape[0]
    pi = rng.permutation(NB)
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[pi], vp2[pi] = kp, vp
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1)
    out2 = decode(q, kp2, vp2, t2, lens, bs, 0.3)
    assert np.array_equal(out.view(np.uint64), out2.view(np.uint64))


def check_sharing_invariance(decode, seed=5):
    """Sequences pointing at shared prefix blocks give bit-identical results to
    the same sequences with private copies (P1 "Diziler Arasında Blokları
    Paylaşma")."""
    rng = np.random.default_rng(seed)
    bs, Hkv, D = 4, 2, 8
    prefix_blocks, NB = 3, 40
    kp = rng.standard_normal((NB, bs, Hkv, D))
    vp = rng.standard_normal((NB, bs, Hkv, D))
    shared = [0, 1, 2]
    tails = [[3, 4], [5], [6, 7]]
    lens = np.array([prefix_blocks * bs + 5, prefix_blocks * bs + 2, prefix_blocks * bs + 8])
    tables = np.full((3, 6), -1)
    for b in range(3):
        row = shared + tails[b]
        tables[b, :len(row)] = row
    q = rng.standard_normal((3, 4, D))
    out = decode(q, kp, vp, tables, lens, bs, 0.4)
    # twin: private copies of the prefix for each sequence
    kp2, vp2 = kp.copy(), vp.copy()
    t2 = tables.copy()
    nxt = 10
    for b in range(3):
        for j in range(prefix_blocks):
            kp2[nxt], vp2[nxt] = kp[shared[j]], vp[shared[j]]
            t2[b, j] = nxt
            nxt += 1
    out2 = decode(q, kp2, vp2, t2, lens, bs, 0.4)
    assert np.array_equal(out.view(np.uint64), out2.view(np.uint64))


# --------------------------------------------------------------------------
# prefill: causal attention of several new tokens per sequence
# --------------------------------------------------------------------------

def random_prefill(rng, Hq, Hkv, D, bs, lens, news):
    """Random pools and scattered tables (float64, poisoned outside the valid
    tokens) plus packed queries for ``news[b]`` new tokens per sequence."""
    B = len(lens)
    _, kp, vp, tables, lens = random_paged(rng, B, Hq, Hkv, D, bs, lens)
    starts = np.concatenate([[0], np.cumsum(news)]).astype(np.int64)
    q = rng.standard_normal((int(starts[-1]), Hq, D))
    return q, kp, vp, tables, lens, starts


def check_prefill_vs_sdpa(prefill, seed=21, Hq=6, Hkv=2, D=8, bs=4, lens=(1, 9, 16, 23), ctx=None):
    """fp64 torch scaled_dot_product_attention on contiguous K/V (explicit slot
    indexing).  Whole prompts (no context) use ``is_causal=True``; prompts
    with ``ctx[b]`` tokens of context use the mask torch.tril(ones, ctx[b]),
    which lets new token i see tokens 0 .. ctx[b] + i."""
    rng = np.random.default_rng(seed)
    ctx = ctx or (0,) * len(lens)
    news = [L - c for L, c in zip(lens, ctx)]
    q, kp, vp, tables, lens, starts = random_prefill(rng, Hq, Hkv, D, bs, lens, news)
    scale = 0.43
    out = prefill(q, kp, vp, tables, lens, starts, bs, scale)
    G = Hq // Hkv
    ks, vs = contiguous(kp, tables, lens, bs), contiguous(vp, tables, lens, bs)
    for b, L in enumerate(lens):
        n = news[b]
        if n == 0:
            continue
        K = torch.from_numpy(ks[b]).permute(1, 0, 2).repeat_interleave(G, dim=0)    # [Hq, L, D]
        V = torch.from_numpy(vs[b]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        Q = torch.from_numpy(q[starts[b]:starts[b + 1]]).permute(1, 0, 2)             # [Hq, n, D]
        if ctx[b] == 0:
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
        else:
            mask = torch.tril(torch.ones(n, int(L), dtype=torch.bool), diagonal=ctx[b])
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
        np.testing.assert_allclose(out[starts[b]:starts[b + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=1e-12, atol=1e-12)


def check_prefill_rows_are_decodes(prefill, decode, seed=22, Hq=4, Hkv=2, D=8, bs=4,
                                   lens=(7, 12, 30), news=(7, 3, 11)):
    """New token i of sequence b at position p gives what a decode step gives
    for a query at the end of the sequence's first p + 1 tokens (the same
    gathered keys and values, no mask), up to rounding order."""
    rng = np.random.default_rng(seed)
    q, kp, vp, tables, lens, starts = random_prefill(rng, Hq, Hkv, D, bs, lens, news)
    scale = 0.29
    out = prefill(q, kp, vp, tables, lens, starts, bs, scale)
    for b in range(len(lens)):
        for i in range(news[b]):
            r = int(starts[b]) + i
            p = int(lens[b]) - news[b] + i
            ref = decode(q[r:r + 1], kp, vp, tables[b:b + 1], np.array([p + 1]), bs, scale)
            np.testing.assert_allclose(out[r], ref[0], rtol=1e-13, atol=1e-13, err_msg=str((b, i)))


def check_prefill_bruteforce(prefill, seed=23, Hq=4, Hkv=2, D=3, bs=3, lens=(4, 8), news=(4, 3)):
    """Pure-Python loops with math.exp over explicit slot indices."""
    rng = np.random.default_rng(seed)
    q, kp, vp, tables, lens, starts = random_prefill(rng, Hq, Hkv, D, bs, lens, news)
    scale = 0.77
    out = prefill(q, kp, vp, tables, lens, starts, bs, scale)
    G = Hq // Hkv
    for b in range(len(lens)):
        for i in range(news[b]):
            r = int(starts[b]) + i
            last = int(lens[b]) - news[b] + i        # the newest token this query may see
            for h in range(Hq):
                g = h // G
                rows = [(int(tables[b, t // bs]), t % bs) for t in range(last + 1)]
                sc = [scale * sum(float(q[r, h, d]) * float(kp[blk, off, g, d]) for d in range(D))
                      for blk, off in rows]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                for d in range(D):
                    ref = sum(wt * float(vp[blk, off, g, d]) for wt, (blk, off) in zip(w, rows)) / sum(w)
                    assert abs(out[r, h, d] - ref) <= 1e-12 * max(1.0, abs(ref)), (b, i, h, d)


def check_prefill_chunking(prefill, seed=24, Hq=4, Hkv=4, D=8, bs=4, lens=(19, 26)):
    """A prompt processed in two chunks (the first with the shorter length,
    the second with the full one) gives the rows of one whole pass, bit for
    bit, whatever the split."""
    rng = np.random.default_rng(seed)
    news = tuple(lens)
    q, kp, vp, tables, lens, starts = random_prefill(rng, Hq, Hkv, D, bs, lens, news)
    whole = prefill(q, kp, vp, tables, lens, starts, bs, 0.5)
    for cut in (1, 5, 12, 18):
        first, second = [], []
        for b in range(len(lens)):
            a = np.arange(int(starts[b]), int(starts[b]) + cut)
            first.append(a)
            second.append(np.arange(int(starts[b]) + cut, int(starts[b + 1])))
        s1 = np.concatenate([[0], np.cumsum([len(a) for a in first])])
        s2 = np.concatenate([[0], np.cumsum([len(a) for a in second])])
        o1 = prefill(q[np.concatenate(first)], kp, vp, tables, np.full(len(lens), cut), s1, bs, 0.5)
        o2 = prefill(q[np.concatenate(second)], kp, vp, tables, lens, s2, bs, 0.5)
        assert np.array_equal(o1, whole[np.concatenate(first)]), cut
        assert np.array_equal(o2, whole[np.concatenate(second)]), cut


def check_prefill_first_token(prefill, seed=25, bs=4, D=8):
    """The first token of a prompt sees only itself, so its output is its own
    value row exactly; a prompt of identical keys averages the value rows it
    sees (closed forms)."""
    rng = np.random.default_rng(seed)
    q, kp, vp, tables, lens, starts = random_prefill(rng, 2, 2, D, bs, (6, 10), (6, 10))
    out = prefill(q, kp, vp, tables, lens, starts, bs, 0.6)
    for b in range(2):
        r = int(starts[b])
        for h in range(2):
            assert np.array_equal(out[r, h], vp[tables[b, 0], 0, h]), (b, h)
    q, kp, vp, tables, lens, starts = random_prefill(rng, 1, 1, D, bs, (9,), (5,))
    for t in range(9):
        kp[tables[0, t // bs], t % bs, 0] = kp[tables[0, 0], 0, 0]
    out = prefill(q, kp, vp, tables, lens, starts, bs, 0.6)
    rows = np.stack([vp[tables[0, t // bs], t % bs, 0] for t in range(9)])
    for i in range(5):
        p = 4 + i
        np.testing.assert_allclose(out[i, 0], rows[:p + 1].mean(axis=0), rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# swap: blocks between a device pool and a host pool
# --------------------------------------------------------------------------

def check_swap_round_trip(swap_blocks, copy_blocks, seed=41):
    """Swapping blocks out to a second pool and back in to fresh places
    leaves their bytes intact (compared as raw bits, NaN patterns included);
    every untouched block of either pool is unchanged; within one pool the
    swap is the copy-on-write block copy; ids outside a pool are skipped."""
    rng = np.random.default_rng(seed)
    dev = rng.integers(0, 2**16, size=(20, 4, 2, 3), dtype=np.uint16)
    host = rng.integers(0, 2**16, size=(12, 4, 2, 3), dtype=np.uint16)
    dev0, host0 = dev.copy(), host.copy()
    out_pairs = np.array([[3, 0], [17, 5], [8, 11], [0, 2]])
    host2 = swap_blocks(dev, host, out_pairs)
    assert np.array_equal(host, host0) and np.array_equal(dev, dev0), "inputs must not change"
    for s_id, d_id in out_pairs:
        assert np.array_equal(host2[d_id], dev[s_id]), (s_id, d_id)
    moved = set(out_pairs[:, 1].tolist())
    for b in range(host.shape[0]):
        if b not in moved:
            assert np.array_equal(host2[b], host[b]), b
    assert np.array_equal(swap_blocks(dev, host, np.zeros((0, 2), dtype=np.int64)), host)
    # back in, to other device blocks
    in_pairs = np.array([[0, 19], [5, 1], [11, 4], [2, 9]])
    dev2 = swap_blocks(host2, dev, in_pairs)
    for (s_out, _), (_, d_in) in zip(out_pairs, in_pairs):
        assert np.array_equal(dev2[d_in], dev[s_out]), (s_out, d_in)
    back = set(in_pairs[:, 1].tolist())
    for b in range(dev.shape[0]):
        if b not in back:
            assert np.array_equal(dev2[b], dev[b]), b
    # one pool: the copy-on-write block copy
    pairs = np.array([[1, 6], [2, 7], [13, 3]])
    assert np.array_equal(swap_blocks(dev, dev, pairs), copy_blocks(dev, pairs))
    # ids outside either pool are skipped
    bad = np.array([[-1, 0], [20, 1], [0, 12], [4, -3], [5, 10]])
    got = swap_blocks(dev, host, bad)
    exp = host.copy()
    exp[10] = dev[5]
    assert np.array_equal(got, exp)


# --------------------------------------------------------------------------
# e4m3 codec
# --------------------------------------------------------------------------

def torch_e4m3_values() -> np.ndarray:
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def check_e4m3_decode(decode_table):
    ref = torch_e4m3_values()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(decode_table), nan)
    assert np.array_equal(decode_table[~nan], ref[~nan])
    assert np.array_equal(np.signbit(decode_table[~nan]), np.signbit(ref[~nan]))


def check_e4m3_encode(encode, decode_table):
    codes = np.arange(256)
    ok = ~np.isnan(decode_table)
    assert np.array_equal(encode(decode_table[ok]), codes[ok].astype(np.uint8))
    # every midpoint between neighbouring positive codes goes to the even code
    vals = decode_table[:0x7F]                       # 0x00 .. 0x7E, increasing
    mids = (vals[:-1] + vals[1:]) / 2.0
    got = encode(mids)
    even = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F))
    assert np.array_equal(got, even.astype(np.uint8)), "ties must round to even"
    assert np.array_equal(encode(-mids), (even | 0x80).astype(np.uint8))
    # just off the midpoints: nearest
    assert np.array_equal(encode(np.nextafter(mids, 0)), np.arange(0x7E).astype(np.uint8))
    assert np.array_equal(encode(np.nextafter(mids, np.inf)), np.arange(1, 0x7F).astype(np.uint8))
    # saturation, infinities, NaN, signed zero
    sat = encode(np.array([448.0, 463.99, 464.0, 464.01, 479.0, 480.0, 1e30, np.inf,
                           -1e30, -np.inf]))
    assert list(sat) == [0x7E] * 8 + [0xFE] * 2, [hex(x) for x in sat]
    assert encode(np.array([np.nan]))[0] == 0x7F
    assert encode(np.array([-np.nan]))[0] == 0xFF
    assert encode(np.array([-0.0]))[0] == 0x80 and encode(np.array([0.0]))[0] == 0x00
    # agreement with torch's cast where torch is defined to saturate-free RNE
    rng = np.random.default_rng(6)
    y = np.concatenate([rng.standard_normal(20000) * 50, rng.uniform(-464, 464, 20000),
                        rng.standard_normal(5000) * 0.01, mids, -mids]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode(y.astype(np.float64)), ref)


def check_e4m3_quantize(quantize):
    """encode(fl32(x * fl32(1/scale))): compare with torch doing the same fp32
    multiply and its own e4m3 cast, inside torch's non-saturating range."""
    rng = np.random.default_rng(7)
    for scale in (0.0117, 0.5, 3.0, 1.0 / 448.0):
        x = rng.standard_normal(4096).astype(np.float32) * np.float32(scale * 300.0)
        inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(scale, dtype=torch.float32)
        y = torch.from_numpy(x) * inv
        keep = y.abs() <= 464
        ref = y[keep].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = quantize(x[keep.numpy()], scale)
        assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# e5m2 codec
# --------------------------------------------------------------------------

def torch_e5m2_values() -> np.ndarray:
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e5m2).to(torch.float64).numpy()


def check_e5m2_decode(decode_table):
    ref = torch_e5m2_values()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(decode_table), nan)
    assert np.array_equal(decode_table[~nan], ref[~nan])
    assert np.array_equal(np.signbit(decode_table[~nan]), np.signbit(ref[~nan]))


def check_e5m2_encode(encode, decode_table):
    codes = np.arange(256)
    finite = np.isfinite(decode_table)
    assert np.array_equal(encode(decode_table[finite]), codes[finite].astype(np.uint8))
    vals = decode_table[:0x7C]                         # 0x00 .. 0x7B, increasing, finite
    mids = (vals[:-1] + vals[1:]) / 2.0
    even = np.where(np.arange(0x7B) % 2 == 0, np.arange(0x7B), np.arange(1, 0x7C))
    assert np.array_equal(encode(mids), even.astype(np.uint8)), "ties must round to even"
    assert np.array_equal(encode(-mids), (even | 0x80).astype(np.uint8))
    assert np.array_equal(encode(np.nextafter(mids, 0)), np.arange(0x7B).astype(np.uint8))
    assert np.array_equal(encode(np.nextafter(mids, np.inf)), np.arange(1, 0x7C).astype(np.uint8))
    sat = encode(np.array([57344.0, 61439.9, 61440.0, 70000.0, np.inf, -np.inf, -1e9]))
    assert list(sat) == [0x7B] * 5 + [0xFB] * 2, [hex(x) for x in sat]
    assert encode(np.array([np.nan]))[0] == 0x7F and encode(np.array([-np.nan]))[0] == 0xFF
    assert encode(np.array([-0.0]))[0] == 0x80 and encode(np.array([0.0]))[0] == 0x00
    # torch's cast (round to nearest even, no saturation) inside the finite range
    rng = np.random.default_rng(8)
    y = np.concatenate([rng.standard_normal(20000) * 3000, rng.uniform(-57344, 57344, 20000),
                        rng.standard_normal(5000) * 1e-4, mids, -mids]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(encode(y.astype(np.float64)), ref)
