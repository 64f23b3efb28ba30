"""Plant plausible mistakes in copies of oracle functions (on the CPU) and
require the pins to catch every one.  This shows the pins are sharp enough
that a dropped term, a wrong sign or index or a swapped operand in the oracle
would not go unnoticed."""

import numpy as np
import pytest

from oracle import blocks, fp8, numerics, paged, sizes
from tests import oracle_pins as pins
from tests import test_oracle_blocks


def decode_with(gmap=None, attend=None, gather=None, length=None):
    """The oracle's decode with one part swapped for a mutant."""
    gmap = gmap or (lambda h, G, Hkv: h // G)
    attend = attend or paged.attend
    gather = gather or paged.gather
    length = length or (lambda L: L)

    def decode(q, kp, vp, tables, lens, bs, scale, seqs=None):
        B, Hq, D = q.shape
        Hkv = kp.shape[2]
        G = Hq // Hkv
        out = np.full((B, Hq, D), np.nan)
        for b in range(B):
            L = length(int(lens[b]))
            kb = gather(kp, tables[b], L, bs)
            vb = gather(vp, tables[b], L, bs)
            for h in range(Hq):
                g = gmap(h, G, Hkv)
                out[b, h] = attend(q[b, h:h + 1], kb[:, g, :], vb[:, g, :], scale)[0]
        return out
    return decode


def attend_no_scale(q, k, v, scale):
    return paged.attend(q, k, v, 1.0)


def attend_wrong_sign(q, k, v, scale):
    return paged.attend(q, k, v, -scale)


def attend_swapped(q, k, v, scale):
    return paged.attend(q, v, k, scale)


def attend_unnormalised(q, k, v, scale):
    s = scale * (q @ k.T)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return w @ v


def attend_no_exp(q, k, v, scale):
    s = scale * (q @ k.T)
    w = s - s.min(axis=1, keepdims=True) + 1e-3
    return (w @ v) / w.sum(axis=1, keepdims=True)


def gather_off_by_one(pool, row, L, bs):
    nb = paged.blocks_for(L, bs)
    ids = np.asarray(row[1:nb + 1], dtype=np.int64)
    ids = np.where(ids < 0, 0, ids)
    return pool[ids].reshape((-1,) + pool.shape[2:])[:L]


def gather_slot_major(pool, row, L, bs):
    nb = paged.blocks_for(L, bs)
    blocks_ = pool[np.asarray(row[:nb], dtype=np.int64)]        # [nb, bs, H, D]
    return blocks_.transpose(1, 0, 2, 3).reshape((nb * bs,) + pool.shape[2:])[:L]


DECODE_MUTANTS = {
    "gqa head modulo": decode_with(gmap=lambda h, G, Hkv: h % Hkv),
    "no softmax scale": decode_with(attend=attend_no_scale),
    "negated scores": decode_with(attend=attend_wrong_sign),
    "K and V swapped": decode_with(attend=attend_swapped),
    "missing normalisation": decode_with(attend=attend_unnormalised),
    "no exponential": decode_with(attend=attend_no_exp),
    "gather off by one block": decode_with(gather=gather_off_by_one),
    "gather slot-major": decode_with(gather=gather_slot_major),
    "drops the newest token": decode_with(length=lambda L: max(L - 1, 0)),
}


def decode_pins(decode):
    pins.check_decode_vs_sdpa(decode)
    pins.check_decode_vs_sdpa(decode, seed=31, B=2, Hq=4, Hkv=2, D=8, bs=4, lens=(9, 6))
    pins.check_decode_vs_bruteforce(decode)
    pins.check_closed_forms(decode)


def test_real_decode_passes_the_same_pins():
    decode_pins(decode_with())
    decode_pins(paged.decode)


@pytest.mark.parametrize("name", sorted(DECODE_MUTANTS))
def test_decode_mutant_is_caught(name):
    with pytest.raises(AssertionError):
        decode_pins(DECODE_MUTANTS[name])


def slot_mapping_swapped(tables, positions, bs):
    out = np.full(len(positions), -1, dtype=np.int32)
    for b, p in enumerate(positions):
        if p >= 0:
            out[b] = tables[b, p % bs] * bs + p // bs
    return out


def write_cache_offset_shift(pool, rows, slots, bs):
    return paged.write_cache(pool, rows, np.where(np.asarray(slots) >= 0, np.asarray(slots) + 1, -1), bs)


def allocate_lifo(pool, length, bs):
    n = -(-length // bs)
    out = []
    for _ in range(n):
        b = pool.free.pop()
        pool.refs[b] = 1
        out.append(b)
    return out


def unused_reserved_wrong(L, reservation):
    return reservation - L + 1


@pytest.mark.parametrize("part", ["slot", "write", "alloc", "reserved"])
def test_worked_example_catches_mutants(part):
    fns = dict(BlockPool=blocks.BlockPool, allocate_sequence=blocks.allocate_sequence,
               slot_mapping=paged.slot_mapping, write_cache=paged.write_cache, gather=paged.gather,
               paged_unused_slots=sizes.paged_unused_slots,
               reserved_unused_slots=sizes.reserved_unused_slots)
    fns.update({"slot": dict(slot_mapping=slot_mapping_swapped),
                "write": dict(write_cache=write_cache_offset_shift),
                "alloc": dict(allocate_sequence=allocate_lifo),
                "reserved": dict(reserved_unused_slots=unused_reserved_wrong)}[part])
    # a mutant may also be caught by running off the table
    with pytest.raises((AssertionError, IndexError)):
        pins.check_worked_example(**fns)


def e4m3_table_bias8():
    t = fp8.DECODE_TABLE.copy()
    return t / 2.0


def encode_half_up(y):
    y = np.asarray(y, dtype=np.float64)
    # round half away from zero instead of half to even
    r = fp8.round_to_e4m3(y)
    lo = fp8.round_to_e4m3(np.nextafter(y, 0))
    tie = (r != lo) & np.isfinite(y)
    bumped = np.where(tie & (np.abs(r) < np.abs(lo)), lo, r)
    return fp8.encode(bumped)


def encode_no_saturation(y):
    y = np.asarray(y, dtype=np.float64)
    out = fp8.encode(y)
    return np.where(np.abs(np.nan_to_num(y, nan=0.0)) > 464.0, np.uint8(0x7F), out).astype(np.uint8)


def encode_truncate(y):
    y = np.asarray(y, dtype=np.float64)
    r = numerics.round_to_format(np.nextafter(y, 0), 4, -6, 448.0, saturate=True)
    return fp8.encode(np.where(np.isfinite(y), r, y))


def test_fp8_mutants_are_caught():
    with pytest.raises(AssertionError):
        pins.check_e4m3_decode(e4m3_table_bias8())
    for enc in (encode_half_up, encode_no_saturation, encode_truncate):
        with pytest.raises(AssertionError):
            pins.check_e4m3_encode(enc, fp8.DECODE_TABLE)


def append_always_copies(pool, table, length, bs):
    pos = int(length)
    if pos % bs == 0:
        table.append(pool.allocate())
        return table[-1] * bs, None
    last = table[pos // bs]
    new = pool.allocate()
    pool.release(last)
    table[pos // bs] = new
    return new * bs + pos % bs, (last, new)


def append_never_copies(pool, table, length, bs):
    pos = int(length)
    if pos % bs == 0:
        table.append(pool.allocate())
    return table[pos // bs] * bs + pos % bs, None


@pytest.mark.parametrize("mutant", [append_always_copies, append_never_copies])
def test_block_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(blocks, "append_slot", mutant)
    with pytest.raises(AssertionError):
        test_oracle_blocks.test_shared_stem_copy_order()


def prefill_with(positions=None, seen=None, gmap=None, rows=None):
    """The oracle's prefill with one part swapped for a mutant: the new
    tokens' positions, how many tokens a query at position p sees, the GQA
    head map, or which q row a new token reads."""
    positions = positions or paged.prefill_positions
    seen = seen or (lambda p, L: p + 1)
    gmap = gmap or (lambda h, G, Hkv: h // G)
    rows = rows or (lambda r0, i, n: r0 + i)

    def prefill(q, kp, vp, tables, lens, starts, bs, scale, seqs=None):
        T, Hq, D = q.shape
        Hkv = kp.shape[2]
        G = Hq // Hkv
        out = np.full((T, Hq, D), np.nan)
        for b in range(len(lens)):
            pos = positions(starts, lens, b)
            L = int(lens[b])
            kb = paged.gather(kp, tables[b], L, bs)
            vb = paged.gather(vp, tables[b], L, bs)
            n = len(pos)
            for i, p in enumerate(pos):
                k = max(1, min(L, seen(int(p), L)))
                for h in range(Hq):
                    g = gmap(h, G, Hkv)
                    out[int(starts[b]) + i, h] = paged.attend(q[rows(int(starts[b]), i, n), h:h + 1],
                                                              kb[:k, g], vb[:k, g], scale)[0]
        return out
    return prefill


def positions_top_left(starts, lens, b):
    return np.arange(int(starts[b + 1]) - int(starts[b]))


PREFILL_MUTANTS = {
    "excludes itself": prefill_with(seen=lambda p, L: p),
    "sees one token ahead": prefill_with(seen=lambda p, L: p + 2),
    "no causal mask": prefill_with(seen=lambda p, L: L),
    "positions from the chunk start": prefill_with(positions=positions_top_left),
    "gqa head modulo": prefill_with(gmap=lambda h, G, Hkv: h % Hkv),
    "rows reversed within a sequence": prefill_with(rows=lambda r0, i, n: r0 + n - 1 - i),
}


def prefill_pins(prefill):
    pins.check_prefill_vs_sdpa(prefill)
    pins.check_prefill_vs_sdpa(prefill, lens=(9, 16, 23, 5), ctx=(8, 3, 10, 0))
    pins.check_prefill_rows_are_decodes(prefill, paged.decode)
    pins.check_prefill_bruteforce(prefill)
    pins.check_prefill_first_token(prefill)


def test_real_prefill_passes_the_same_pins():
    prefill_pins(prefill_with())
    prefill_pins(paged.prefill)


@pytest.mark.parametrize("name", sorted(PREFILL_MUTANTS))
def test_prefill_mutant_is_caught(name):
    with pytest.raises(AssertionError):
        prefill_pins(PREFILL_MUTANTS[name])


def swap_shifted(src, dst, pairs):
    return paged.swap_blocks(src, dst, np.asarray(pairs)[:, ::-1] if len(pairs) else pairs)


def swap_no_bounds(src, dst, pairs):
    out = np.array(dst, copy=True)
    for s_id, d_id in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        out[int(d_id) % out.shape[0]] = src[int(s_id) % src.shape[0]]
    return out


def swap_in_place(src, dst, pairs):
    out = np.asarray(dst)        # forgets to copy: the caller's array changes
    for s_id, d_id in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if 0 <= s_id < src.shape[0] and 0 <= d_id < out.shape[0]:
            out[int(d_id)] = src[int(s_id)]
    return out


@pytest.mark.parametrize("mutant", [swap_shifted, swap_no_bounds, swap_in_place])
def test_swap_mutants_are_caught(mutant):
    with pytest.raises((AssertionError, IndexError)):
        pins.check_swap_round_trip(mutant, paged.copy_blocks)


def e5m2_encode_truncate(y):
    y = np.asarray(y, dtype=np.float64)
    r = numerics.round_to_format(np.nextafter(y, 0), 3, -14, 57344.0, saturate=True)
    return fp8.encode_e5m2(np.where(np.isfinite(y), r, y))


def e5m2_encode_overflow_to_inf(y):
    y = np.asarray(y, dtype=np.float64)
    out = fp8.encode_e5m2(y)
    big = np.abs(np.nan_to_num(y, nan=0.0)) > 61440.0
    return np.where(big, np.where(y > 0, np.uint8(0x7C), np.uint8(0xFC)), out).astype(np.uint8)


def test_e5m2_mutants_are_caught():
    with pytest.raises(AssertionError):
        pins.check_e5m2_decode(fp8.DECODE_TABLE_E5M2 * 2.0)
    for enc in (e5m2_encode_truncate, e5m2_encode_overflow_to_inf):
        with pytest.raises(AssertionError):
            pins.check_e5m2_encode(enc, fp8.DECODE_TABLE_E5M2)
