"""Pins of the CPU oracle against the pages, closed forms, library routines and brute force."""

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import blocks, fp8, numerics, paged, sizes
from tests import oracle_pins as pins


# ---------------------------------------------------------------- worked example

def test_worked_example_from_the_code_sketch():
    pins.check_worked_example(blocks.BlockPool, blocks.allocate_sequence, paged.slot_mapping,
                              paged.write_cache, paged.gather, sizes.paged_unused_slots,
                              sizes.reserved_unused_slots)


# ---------------------------------------------------------------- size figures

def test_size_figures_printed_by_the_pages():
    g = pins.load_golden("size_figures.json")
    for f in g["figures"]:
        m = f["model"]
        got = sizes.kv_bytes(f["tokens"], m["layers"], m["kv_heads"], m["head_dim"], m["elem_bytes"]) / 1e9
        assert abs(got - f["value"]) <= f["rel_tol"] * f["value"], (f["what"], got)
    assert sizes.kv_bytes_per_token(40, 40, 128, 2) == 819_200       # 13B: 2*40*5120*2
    assert sizes.kv_bytes_per_token(80, 8, 128, 2) == 327_680        # 70B GQA
    w = g["waste"]
    assert round(100 * sizes.waste_fraction(w[0]["used"], w[0]["reserved"])) == w[0]["percent_wasted"]
    assert sizes.reserved_unused_slots(w[1]["used"], w[1]["reserved"]) == w[1]["slots_wasted"]


def test_paged_waste_is_below_one_block():
    for L in range(1, 200):
        u = sizes.paged_unused_slots(L, 16)
        assert 0 <= u < 16 and (L + u) % 16 == 0


# ---------------------------------------------------------------- attention

def test_decode_matches_torch_sdpa_fp64():
    pins.check_decode_vs_sdpa(paged.decode)
    pins.check_decode_vs_sdpa(paged.decode, seed=11, B=2, Hq=4, Hkv=4, D=8, bs=16, lens=(16, 33))
    pins.check_decode_vs_sdpa(paged.decode, seed=12, B=2, Hq=8, Hkv=1, D=8, bs=2, lens=(5, 1))


@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 10_000), G=st.sampled_from([1, 2, 4]), Hkv=st.integers(1, 3),
       bs=st.sampled_from([1, 2, 4, 16]), lens=st.lists(st.integers(0, 40), min_size=1, max_size=4))
def test_decode_matches_sdpa_random_shapes(seed, G, Hkv, bs, lens):
    if max(lens) == 0:
        lens = lens + [1]
    lens = [L for L in lens]
    nonzero = [L for L in lens if L > 0]
    pins.check_decode_vs_sdpa(paged.decode, seed=seed, B=len(nonzero), Hq=G * Hkv, Hkv=Hkv, D=8,
                              bs=bs, lens=tuple(nonzero))


def test_decode_matches_bruteforce_loops():
    pins.check_decode_vs_bruteforce(paged.decode)
    pins.check_decode_vs_bruteforce(paged.decode, seed=21, B=3, Hq=3, Hkv=1, D=4, bs=2, lens=(1, 4, 7))


def test_decode_closed_forms():
    pins.check_closed_forms(paged.decode)


def test_decode_placement_invariance_bit_exact():
    pins.check_placement_invariance(paged.decode)


def test_decode_sharing_invariance_bit_exact():
    pins.check_sharing_invariance(paged.decode)


def test_decode_never_reads_poisoned_slots():
    rng = np.random.default_rng(8)
    q, kp, vp, tables, lens = pins.random_paged(rng, 3, 4, 2, 8, 4, (5, 9, 4), poison=True)
    out = paged.decode(q, kp, vp, tables, lens, 4, 0.3)
    assert np.isfinite(out).all()


def test_decode_subset_of_sequences():
    rng = np.random.default_rng(9)
    q, kp, vp, tables, lens = pins.random_paged(rng, 4, 4, 2, 8, 4, (5, 9, 4, 2))
    full = paged.decode(q, kp, vp, tables, lens, 4, 0.3)
    part = paged.decode(q, kp, vp, tables, lens, 4, 0.3, seqs=[1, 3])
    assert np.array_equal(full[[1, 3]], part[[1, 3]])
    assert np.isnan(part[[0, 2]]).all()


# ---------------------------------------------------------------- slot mapping / write / copy

def test_slot_mapping_enumerates_every_slot():
    rng = np.random.default_rng(10)
    bs, NB = 4, 30
    perm = rng.permutation(NB)
    tables = np.stack([perm[:5], perm[5:10], perm[10:15]]).astype(np.int32)
    for b in range(3):
        for pos in range(5 * bs):
            s = paged.slot_mapping(tables, np.array([-1] * b + [pos] + [-1] * (2 - b)), bs)
            assert s[b] == tables[b, pos // bs] * bs + pos % bs
            assert all(s[i] == -1 for i in range(3) if i != b)
    # every (sequence, position) gets a distinct slot
    seen = set()
    for b in range(3):
        for pos in range(5 * bs):
            seen.add(int(paged.slot_mapping(tables[b:b + 1], np.array([pos]), bs)[0]))
    assert len(seen) == 3 * 5 * bs


def test_write_cache_touches_only_its_slots():
    rng = np.random.default_rng(12)
    pool = rng.integers(0, 2 ** 16, size=(6, 4, 2, 8), dtype=np.uint16)
    rows = rng.integers(0, 2 ** 16, size=(3, 2, 8), dtype=np.uint16)
    slots = np.array([5, -1, 22])
    out = paged.write_cache(pool, rows, slots, 4)
    ref = pool.copy()
    ref[1, 1] = rows[0]
    ref[5, 2] = rows[2]
    assert np.array_equal(out, ref)


def test_copy_blocks_whole_block_bytes():
    rng = np.random.default_rng(13)
    pool = rng.integers(0, 256, size=(8, 4, 2, 8), dtype=np.uint8)
    out = paged.copy_blocks(pool, np.array([[1, 5], [1, 6], [3, 0]]))
    ref = pool.copy()
    ref[5], ref[6], ref[0] = pool[1], pool[1], pool[3]
    assert np.array_equal(out, ref)


# ---------------------------------------------------------------- numerics

def test_bits_to_f64_match_torch():
    rng = np.random.default_rng(14)
    bits16 = rng.integers(0, 2 ** 16, size=50000, dtype=np.uint16)
    ref_bf = torch.from_numpy(bits16.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got_bf = numerics.bf16_bits_to_f64(bits16)
    same = (got_bf == ref_bf) | (np.isnan(got_bf) & np.isnan(ref_bf))
    assert same.all()
    ref_h = torch.from_numpy(bits16.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    got_h = numerics.f16_bits_to_f64(bits16)
    assert ((got_h == ref_h) | (np.isnan(got_h) & np.isnan(ref_h))).all()


def test_round_to_f16_and_f32_match_numpy_casts():
    rng = np.random.default_rng(15)
    x = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.integers(-9, 6, 50000),
                        [65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -25, 2.0 ** -24, 0.0, -0.0]])
    # every tie between neighbouring fp16 values in a few binades
    h = np.arange(0, 2 ** 15, dtype=np.uint16).view(np.float16).astype(np.float64)
    h = h[np.isfinite(h)]
    ties = (h[:-1] + h[1:]) / 2
    x = np.concatenate([x, ties, -ties])
    got = numerics.round_to_f16(x)
    ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    got32 = numerics.round_to_f32(x)
    assert np.array_equal(got32, x.astype(np.float32).astype(np.float64))


def test_round_to_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(16)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)).astype(np.float32)
    b = np.arange(0, 2 ** 15, 7, dtype=np.uint32) << 16
    bv = b.view(np.float32).astype(np.float64)
    bv = bv[np.isfinite(bv)]
    ties = ((bv[:-1] + bv[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = numerics.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_half_ulp_closed_forms():
    assert numerics.half_ulp(1.0, 11, -14) == 2.0 ** -11
    assert numerics.half_ulp(4.5, 8, -126) == 2.0 ** -6
    assert numerics.half_ulp(0.0, 11, -14) == 2.0 ** -25


# ---------------------------------------------------------------- fp8

def test_e4m3_decode_matches_torch_all_codes():
    pins.check_e4m3_decode(fp8.DECODE_TABLE)


def test_e4m3_decode_named_values():
    t = fp8.DECODE_TABLE
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6 and t[0x38] == 1.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])


def test_e4m3_encode_rne_saturating():
    pins.check_e4m3_encode(fp8.encode, fp8.DECODE_TABLE)


def test_e4m3_quantize_fp32_multiply():
    pins.check_e4m3_quantize(fp8.quantize)


# ---------------------------------------------------------------- blocks

def test_out_of_blocks_raises():
    pool = blocks.BlockPool(free=[3])
    blocks.allocate_sequence(pool, 16, 16)
    with pytest.raises(blocks.OutOfBlocks):
        blocks.allocate_sequence(pool, 1, 16)


# ---------------------------------------------------------------- prefill

def test_prefill_whole_prompts_match_causal_sdpa():
    pins.check_prefill_vs_sdpa(paged.prefill)
    pins.check_prefill_vs_sdpa(paged.prefill, seed=31, Hq=8, Hkv=1, D=16, bs=16, lens=(40, 17, 3))


def test_prefill_with_context_matches_masked_sdpa():
    pins.check_prefill_vs_sdpa(paged.prefill, lens=(9, 16, 23, 5), ctx=(8, 3, 10, 0))
    pins.check_prefill_vs_sdpa(paged.prefill, seed=32, Hq=4, Hkv=4, D=8, bs=2, lens=(33, 12),
                               ctx=(20, 11))


def test_prefill_rows_are_decode_steps():
    pins.check_prefill_rows_are_decodes(paged.prefill, paged.decode)


def test_prefill_bruteforce():
    pins.check_prefill_bruteforce(paged.prefill)


def test_prefill_chunking_and_closed_forms():
    pins.check_prefill_chunking(paged.prefill)
    pins.check_prefill_first_token(paged.prefill)


@settings(max_examples=20, deadline=None)
@given(seed=st.integers(0, 10_000), G=st.sampled_from([1, 2, 4]), Hkv=st.integers(1, 2),
       bs=st.sampled_from([1, 4, 16]), lens=st.lists(st.integers(1, 30), min_size=1, max_size=3),
       frac=st.floats(0.0, 1.0))
def test_prefill_matches_sdpa_random_shapes(seed, G, Hkv, bs, lens, frac):
    ctx = tuple(int(frac * (L - 1)) for L in lens)
    pins.check_prefill_vs_sdpa(paged.prefill, seed=seed, Hq=G * Hkv, Hkv=Hkv, D=8, bs=bs,
                               lens=tuple(lens), ctx=ctx)


# ---------------------------------------------------------------- swap

def test_swap_blocks_round_trip():
    pins.check_swap_round_trip(paged.swap_blocks, paged.copy_blocks)


# ---------------------------------------------------------------- e5m2

def test_e5m2_decode_matches_torch():
    pins.check_e5m2_decode(fp8.DECODE_TABLE_E5M2)


def test_e5m2_encode_round_trip_ties_and_saturation():
    pins.check_e5m2_encode(fp8.encode_e5m2, fp8.DECODE_TABLE_E5M2)


def test_e5m2_quantize_matches_torch():
    rng = np.random.default_rng(9)
    for scale in (0.01, 0.5, 3.0):
        x = rng.standard_normal(4096).astype(np.float32) * np.float32(scale * 20000.0)
        inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(scale, dtype=torch.float32)
        yt = torch.from_numpy(x) * inv
        keep = yt.abs() <= 57344
        ref = yt[keep].to(torch.float8_e5m2).view(torch.uint8).numpy()
        assert np.array_equal(fp8.quantize_e5m2(x[keep.numpy()], scale), ref)
