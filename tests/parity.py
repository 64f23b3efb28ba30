"""Oracle expectations for one decode step, and the comparisons the GPU
parity tests make.

Everything expected here comes from the oracle applied to the step's inputs
(the pre-step state from the seeded generator); nothing the GPU produced is
fed back into the oracle.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from oracle import blocks as oblocks
from oracle import fp8, numerics, paged

#: attention tolerance (max abs error vs the fp64 oracle) by KV dtype; the
#: output rounding (half an ulp of the output dtype) is added on top.
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2, "e4m3": 3e-2, "e5m2": 3e-2}
OUT_FORMAT = {"f32": (numerics.F32_P, numerics.F32_EMIN), "f16": (numerics.F16_P, numerics.F16_EMIN),
              "bf16": (numerics.BF16_P, numerics.BF16_EMIN)}


def storage(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a tensor as a NumPy array (uint32 / uint16 / uint8)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.numpy()
    raise TypeError(t.dtype)


def widen(raw: np.ndarray, dtype: str, scale=1.0) -> np.ndarray:
    """Raw storage to float64 values; for 8-bit codes ``scale`` is the pool's
    fp32 scale, or an array of one scale per KV head for ``raw`` shaped
    [..., Hkv, D]."""
    if np.ndim(scale) > 0:
        per = np.asarray(scale, dtype=np.float32).astype(np.float64)[:, None]
        return widen(raw, dtype, 1.0) * per
    return _widen(raw, dtype, scale)


def _widen(raw: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    if dtype == "f32":
        return numerics.f32_bits_to_f64(raw)
    if dtype == "f16":
        return numerics.f16_bits_to_f64(raw)
    if dtype == "bf16":
        return numerics.bf16_bits_to_f64(raw)
    if dtype == "e4m3":
        return fp8.decode(raw, scale)
    if dtype == "e5m2":
        return fp8.decode_e5m2(raw, scale)
    raise ValueError(dtype)


def encode_rows(rows: np.ndarray, src_dtype: str, kv_dtype: str, scale: float) -> np.ndarray:
    """The oracle's cache-write encoding of new rows (raw storage in, raw out)."""
    if src_dtype == kv_dtype:
        return rows
    quant = fp8.quantize_e5m2 if kv_dtype == "e5m2" else fp8.quantize
    if np.ndim(scale) > 0:          # one scale per KV head: rows [T, Hkv, D]
        vals = widen(rows, src_dtype)
        out = np.empty(rows.shape, dtype=np.uint8)
        for h in range(rows.shape[1]):
            out[:, h, :] = quant(vals[:, h, :], float(scale[h]))
        return out
    return quant(widen(rows, src_dtype), scale)


@dataclass
class PreStep:
    """Host copies of a workload's inputs, taken before the GPU step runs."""

    k_pool: np.ndarray
    v_pool: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    q: np.ndarray


def snapshot(wl) -> PreStep:
    return PreStep(storage(wl.k_pool), storage(wl.v_pool), storage(wl.k_new), storage(wl.v_new),
                   storage(wl.q))


@dataclass
class Expected:
    tables: list
    copies: list
    slots: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    out: np.ndarray       # float64, NaN rows for sequences not computed


def oracle_step(wl, pre: PreStep, seqs=None) -> Expected:
    cfg = wl.cfg
    bs = cfg.block_size
    pool = oblocks.BlockPool(free=list(wl.free), refs=dict(wl.refs))
    tables = [list(r) for r in wl.tables]
    copies = []
    for i, L in enumerate(wl.seq_lens):
        if L >= 1:
            _, cow = oblocks.append_slot(pool, tables[i], int(L) - 1, bs)
            if cow is not None:
                copies.append(cow)
    width = max(1, max(len(r) for r in tables))
    tab = np.full((len(tables), width), -1, dtype=np.int64)
    for i, r in enumerate(tables):
        tab[i, :len(r)] = r
    positions = np.where(wl.seq_lens > 0, wl.seq_lens - 1, -1)
    slots = paged.slot_mapping(tab, positions, bs)

    def enc(rows, scale):
        return encode_rows(rows, cfg.src_dtype, cfg.kv_dtype, scale)

    k = paged.copy_blocks(pre.k_pool, np.array(copies).reshape(-1, 2))
    v = paged.copy_blocks(pre.v_pool, np.array(copies).reshape(-1, 2))
    k = paged.write_cache(k, enc(pre.k_new, wl.k_scale), slots, bs)
    v = paged.write_cache(v, enc(pre.v_new, wl.v_scale), slots, bs)
    q = widen(pre.q, cfg.q_dtype)
    out = paged.decode(q, k, v, tab, wl.seq_lens, bs, wl.scale, seqs=seqs,
                       widen_k=lambda x: widen(x, cfg.kv_dtype, wl.k_scale),
                       widen_v=lambda x: widen(x, cfg.kv_dtype, wl.v_scale))
    return Expected(tables, copies, slots, k, v, out)


@dataclass
class PrefillExpected:
    slots: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    out: np.ndarray       # float64 [T, Hq, D], NaN rows for sequences not computed


def prefill_row_tables(tables: np.ndarray, q_starts: np.ndarray) -> np.ndarray:
    """The table row of the sequence owning each new row (for slot mapping)."""
    owner = np.repeat(np.arange(len(q_starts) - 1), np.diff(q_starts))
    return tables[owner]


def prefill_table(wl) -> np.ndarray:
    width = max(1, max(len(r) for r in wl.tables))
    tab = np.full((len(wl.tables), width), -1, dtype=np.int64)
    for i, r in enumerate(wl.tables):
        tab[i, :len(r)] = r
    return tab


def prefill_slots(wl) -> np.ndarray:
    """The oracle's slot of every new row: its sequence's table row at the
    row's position."""
    tab = prefill_table(wl)
    positions = np.concatenate([paged.prefill_positions(wl.q_starts, wl.seq_lens, b)
                                for b in range(len(wl.seq_lens))] or [np.zeros(0, np.int64)])
    return paged.slot_mapping(prefill_row_tables(tab, wl.q_starts), positions, wl.cfg.block_size)


def oracle_prefill(wl, pre: PreStep, seqs=None) -> PrefillExpected:
    cfg = wl.cfg
    bs = cfg.block_size
    tab = prefill_table(wl)
    slots = prefill_slots(wl)

    def enc(rows, scale):
        return encode_rows(rows, cfg.src_dtype, cfg.kv_dtype, scale)

    k = paged.write_cache(pre.k_pool, enc(pre.k_new, wl.k_scale), slots, bs)
    v = paged.write_cache(pre.v_pool, enc(pre.v_new, wl.v_scale), slots, bs)
    q = widen(pre.q, cfg.q_dtype)
    out = paged.prefill(q, k, v, tab, wl.seq_lens, wl.q_starts, bs, wl.scale, seqs=seqs,
                        widen_k=lambda x: widen(x, cfg.kv_dtype, wl.k_scale),
                        widen_v=lambda x: widen(x, cfg.kv_dtype, wl.v_scale))
    return PrefillExpected(slots, k, v, out)


def gpu_out(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, kv_dtype: str, out_dtype: str, what=""):
    """|got - ref| <= TOL[kv] + half an ulp of the output dtype at ref."""
    p, emin = OUT_FORMAT[out_dtype]
    bound = TOL[kv_dtype] + numerics.half_ulp(ref, p, emin)
    err = np.abs(got - ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; max err "
                             f"{np.nanmax(err):.3e}; first {idx.tolist()} got "
                             f"{got[tuple(idx[0])]} ref {ref[tuple(idx[0])]}")
    return float(np.max(err)) if err.size else 0.0
