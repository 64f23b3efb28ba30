"""The paged KV cache and decode attention, restated plainly in float64
(test infrastructure only).

Layout: a K pool and a V pool, each ``[num_blocks, block_size, Hkv, D]``.
P1's code sketch ("Sayfalama Nasıl Çalışır") uses one head,
``[num_blocks, block_size, head_dim]``; the head axis after the slot axis is
the reading used throughout.  A sequence's block table lists, in logical
order, the physical blocks that hold its tokens (P1 introduction and
"Sayfalama Nasıl Çalışır"; P3 article B "راه حل: PagedAttention", the page
table).  Only the first ceil(L / block_size) entries of a table row mean
anything; the rest, and the slots after token L-1 in the last block, are never
read.

Functions here work on NumPy arrays.  Storage arrays (pools, new rows) may hold
raw bit patterns of any dtype -- the cache write and the block copy only move
them.  Attention takes pools already widened to float64 (see
:mod:`oracle.numerics` and :mod:`oracle.fp8`).
"""

from __future__ import annotations

import numpy as np


def blocks_for(length: int, block_size: int) -> int:
    """Number of blocks a sequence of ``length`` tokens occupies: ceil(L / bs)
    (P1 code sketch: a 40-token request needs ceil(40/16) = 3 blocks)."""
    return -(-int(length) // int(block_size))


def slot_mapping(block_tables: np.ndarray, positions: np.ndarray, block_size: int) -> np.ndarray:
    """Flat slot of the token at ``positions[b]`` of sequence ``b``.

    P1 "Sayfalama Nasıl Çalışır" (code sketch, write loop): the token at
    position ``pos`` goes to physical block ``table[pos // bs]`` at offset
    ``pos % bs``; the flat slot is ``block * bs + offset``.  A negative
    position means "no token" and maps to slot -1.

    Pinned by the worked example (tests/golden/worked_example.json) and by
    brute-force enumeration of every slot of random tables.
    """
    tables = np.asarray(block_tables, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    out = np.full(pos.shape, -1, dtype=np.int64)
    for b in range(pos.shape[0]):
        p = int(pos[b])
        if p < 0:
            continue
        block = int(tables[b, p // block_size])
        out[b] = block * block_size + p % block_size
    return out.astype(np.int32)


def write_cache(pool: np.ndarray, rows: np.ndarray, slots: np.ndarray, block_size: int) -> np.ndarray:
    """Return a copy of ``pool`` with ``rows[i]`` stored at flat slot ``slots[i]``.

    P1 "Sayfalama Nasıl Çalışır" (code sketch, write loop): each new row lands
    at block ``slot // bs``, offset ``slot % bs``.  ``rows`` is
    ``[T, Hkv, D]`` already in the pool's storage encoding; slots < 0 are
    skipped.  Every other byte of the pool is unchanged.
    """
    out = np.array(pool, copy=True)
    for i, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        out[int(s) // block_size, int(s) % block_size] = rows[i]
    return out


def copy_blocks(pool: np.ndarray, pairs: np.ndarray) -> np.ndarray:
    """Return a copy of ``pool`` with whole block ``src`` copied over ``dst``
    for every ``(src, dst)`` row of ``pairs``.

    P1 "Diziler Arasında Blokları Paylaşma": before a sequence writes into a
    block that other sequences still reference, the block is copied
    (copy-on-write); P3 article A names the same step.  The whole block moves,
    unused tail slots included.  Precondition (the pages are silent): the dst
    blocks are distinct and no dst is also a src, so the order of the pairs
    does not matter; every copy reads the pool as it was before the call.
    """
    before = np.asarray(pool)
    out = np.array(pool, copy=True)
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        out[int(dst)] = before[int(src)]
    return out


def swap_blocks(src_pool: np.ndarray, dst_pool: np.ndarray, pairs: np.ndarray) -> np.ndarray:
    """Return a copy of ``dst_pool`` with whole block ``src`` of ``src_pool``
    copied over block ``dst`` for every ``(src, dst)`` row of ``pairs``.

    P3 article A names page-granular eviction: single pages move between GPU
    memory and CPU memory instead of whole sequences.  Moving a page out is
    this copy from the device pool to a host pool, moving it back in is the
    copy the other way; every byte of the block moves, unused tail slots
    included.  Pairs naming a block outside either pool are skipped (a
    reading; the pages are silent).  Precondition: the dst ids are distinct.
    """
    src = np.asarray(src_pool)
    out = np.array(dst_pool, copy=True)
    for s_id, d_id in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if not (0 <= s_id < src.shape[0] and 0 <= d_id < out.shape[0]):
            continue
        out[int(d_id)] = src[int(s_id)]
    return out


def gather(pool: np.ndarray, table_row: np.ndarray, length: int, block_size: int) -> np.ndarray:
    """A sequence's cache as a contiguous ``[L, Hkv, D]`` array.

    P1 "Sayfalama Nasıl Çalışır" (code sketch, read-back): index the pool by
    the sequence's block table, flatten blocks and slots into one token axis
    and keep the first L tokens.  Only the first ceil(L / bs) table entries
    are touched.
    """
    nb = blocks_for(length, block_size)
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    blocks = pool[ids]                                   # [nb, bs, Hkv, D]
    return blocks.reshape((nb * block_size,) + pool.shape[2:])[:length]


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of query rows ``q [G, D]`` over one head's contiguous
    keys ``k [L, D]`` and values ``v [L, D]``, float64.

    The pages never print the attention formula; the reading is standard
    scaled dot-product attention (P1 "İlgili Teknikler" says the kernels are
    FlashAttention-style, i.e. exact attention computed in tiles):
    ``s_t = scale * q . k_t``, ``w_t = exp(s_t - max s)``,
    ``out = sum_t w_t v_t / sum_t w_t``.  A decode query sees its whole
    context, so there is no mask.  L = 0 gives zeros (a reading; the pages are
    silent).

    Pinned against torch's scaled_dot_product_attention in float64, against a
    pure-Python triple loop, and by closed forms (L = 1, q = 0, a planted
    dominant key).
    """
    q = np.asarray(q, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    s = float(scale) * (q @ k.T)                       # [G, L]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    return (w @ v) / w.sum(axis=1, keepdims=True)


def decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_tables: np.ndarray,
           seq_lens: np.ndarray, block_size: int, scale: float, seqs=None,
           widen_k=None, widen_v=None) -> np.ndarray:
    """Paged decode attention for a batch, float64.

    ``q [B, Hq, D]``; pools ``[NB, bs, Hkv, D]`` float64 (already dequantised);
    ``block_tables [B, max_blocks]``; ``seq_lens [B]``.  For each sequence the
    cache is gathered through its block table (P1 "Sayfalama Nasıl Çalışır":
    the attention kernel follows the table block by block) and every query
    head attends over it.  Grouped-query attention (P1 "İlgili Teknikler")
    shares each KV head among G = Hq / Hkv query heads; the reading is that
    consecutive query heads share one: head h uses KV head h // G.

    ``seqs`` restricts the work to some sequence indices; the other rows of
    the result are NaN.  ``widen_k`` / ``widen_v`` map a gathered block of
    raw storage to float64 values (e.g. bf16 bits, or e4m3 codes times the
    pool's scale), so pools can be passed in their storage form and only
    the gathered tokens are widened.
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    out = np.full((B, Hq, D), np.nan, dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        kb = gather(k_pool, block_tables[b], L, block_size)   # [L, Hkv, D]
        vb = gather(v_pool, block_tables[b], L, block_size)
        kb = np.asarray(kb, dtype=np.float64) if widen_k is None else widen_k(kb)
        vb = np.asarray(vb, dtype=np.float64) if widen_v is None else widen_v(vb)
        for g in range(Hkv):
            out[b, g * G:(g + 1) * G] = attend(q[b, g * G:(g + 1) * G], kb[:, g, :], vb[:, g, :], scale)
    return out


def prefill_positions(q_starts: np.ndarray, seq_lens: np.ndarray, b: int):
    """Positions of sequence ``b``'s new tokens: the last n = q_starts[b+1] -
    q_starts[b] of its seq_lens[b] tokens, i.e. L - n, ..., L - 1.

    The tokens before them (L - n of them) are context already in the cache:
    an earlier chunk of the same prompt, or prefix blocks shared with other
    requests (P1 "Diziler Arasında Blokları Paylaşma", prompt caching).
    """
    n = int(q_starts[b + 1]) - int(q_starts[b])
    L = int(seq_lens[b])
    return np.arange(L - n, L, dtype=np.int64)


def prefill(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_tables: np.ndarray,
            seq_lens: np.ndarray, q_starts: np.ndarray, block_size: int, scale: float,
            seqs=None, widen_k=None, widen_v=None) -> np.ndarray:
    """Paged prefill attention for a batch (several new tokens per sequence),
    float64.

    ``q [T, Hq, D]`` packs the new tokens of all sequences: sequence b owns
    rows ``q_starts[b] .. q_starts[b+1]-1``.  Their keys and values are
    already in the pools, so sequence b's context holds ``seq_lens[b]``
    tokens, the new ones last (:func:`prefill_positions`).  A new token at
    position p attends to tokens 0..p of its sequence and to nothing later:
    the model caches the keys and values of previous tokens for the next
    ones (P1 "Çözdüğü Bellek Sorunu"), so a token sees itself and its past
    (the causal reading; the pages print no mask).  Keys and values are
    gathered through the block table (P1 "Sayfalama Nasıl Çalışır") and
    each new token is attended exactly as :func:`attend` attends a decode
    query over the first p + 1 tokens (P1 "İlgili Teknikler": the
    FlashAttention-style kernels of current engines read paged blocks).
    Grouped-query heads map as in :func:`decode`.

    ``seqs`` restricts the work to some sequence indices (other rows NaN);
    ``widen_k`` / ``widen_v`` as in :func:`decode`.
    """
    T, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    B = len(seq_lens)
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        pos = prefill_positions(q_starts, seq_lens, b)
        if pos.size == 0:
            continue
        if pos[0] < 0:
            raise ValueError("a sequence has more new tokens than tokens")
        L = int(seq_lens[b])
        kb = gather(k_pool, block_tables[b], L, block_size)
        vb = gather(v_pool, block_tables[b], L, block_size)
        kb = np.asarray(kb, dtype=np.float64) if widen_k is None else widen_k(kb)
        vb = np.asarray(vb, dtype=np.float64) if widen_v is None else widen_v(vb)
        r0 = int(q_starts[b])
        for i, p in enumerate(pos):
            seen = int(p) + 1
            for g in range(Hkv):
                heads = slice(g * G, (g + 1) * G)
                out[r0 + i, heads] = attend(q[r0 + i, heads], kb[:seen, g, :], vb[:seen, g, :], scale)
    return out
