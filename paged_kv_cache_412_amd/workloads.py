"""Seeded synthetic inputs for the paged decode path.

This module makes inputs only: shapes, sequence lengths, scattered block
tables, pool contents, new K/V rows and queries.  It holds none of the path's
arithmetic (no slot computation, no attention, no quantiser of its own), so the
GPU library and the CPU oracle can both be fed from it.

Workloads (shapes follow the pages' examples; P1 = Ultralytics glossary page
"PagedAttention", P3 = gyaansetu.com page on KV memory and PagedAttention):

* ``tiny``   -- 4 sequences of {40, 17, 64, 1} tokens, 8 heads, head dim 64,
  block size 16 (P1 "Sayfalama Nasıl Çalışır": the default block size, and the
  40-token request of the code sketch), fp32, a pool of 64 blocks.
* ``llama13b`` -- a LLaMA-13B-shaped layer (P1 "Çözdüğü Bellek Sorunu"): 40 heads,
  head dim 128, fp16, batch 64, lengths uniform in [128, 2048].
* ``llama70b`` -- a Llama-3.1-70B-shaped GQA layer (P3 article A, the memory
  problem): 64 query / 8 KV heads, head dim 128, bf16, batch 256, 4,096
  tokens each.
* ``shared`` -- shared-prefix parallel sampling (P1 "Diziler Arasında Blokları
  Paylaşma"): 32 prompts x 3 samples, a 1,024-token prefix held once,
  per-prompt stems of 64..512 tokens shared by the 3 samples, 40 heads,
  head dim 128, fp16.
* ``long_fp8`` / ``long_fp8_bs32`` -- long context with an e4m3 cache and one
  fp32 scale per pool (P1 "İlgili Teknikler": GQA and FP8 cache), 32 query /
  8 KV heads, head dim 128, batch 16, lengths uniform in [16384, 32768],
  block size 16 or 32, bf16 queries and new rows.  ``long_e5m2`` is the same
  with an e5m2 cache (the other 8-bit flavour); ``long_fp8_heads`` uses one
  scale per KV head, with head magnitudes spread over 2^-4..2^4.

Prefill workloads (several new tokens per sequence, :func:`make_prefill`):

* ``prefill13b`` -- the 13B layer shape, 16 whole prompts of 512..4096
  tokens (no cached context), fp16.
* ``prefill70b`` -- the 70B GQA shape, 16 chunks of 1,024 new tokens after
  0..3072 cached tokens (chunked prefill, or a prompt behind a cached
  prefix), bf16.
* ``prefill_fp8`` -- GQA 32/8 with an e4m3 cache, 8 chunks of 2,048 new
  tokens after 0..6144 cached tokens, bf16 queries.

Request stream (:func:`make_stream`): ``prefix_stream`` -- continuous
batching of 3,000 requests, at most 256 sequences at once; 80 % of prompts
start with one of 8 system prompts of 256..2048 tokens (P1 "Diziler Arasında
Blokları Paylaşma": requests with the same system prompt), then 16..256 user
tokens; a quarter ask for 3 samples that share the prompt (P1 "İlgili
Teknikler": a request with n=3); each sequence generates 32..256 tokens and is
freed when done.

Swap workload (:func:`make_swap`): ``swap13b`` -- 1,024 blocks of the 13B
layer's shape (16 tokens x 40 heads x 128, fp16: 160 KiB per block and pool)
evicted to a pinned host pool and restored to other device blocks (P3
article A: pages move to CPU memory one at a time).

State handed to the step (the "pre-step" state): every sequence's cache holds
its first L-1 tokens; the decode step appends token L-1 and then attends over
all L tokens.  Tables hold ceil((L-1)/bs) blocks; the host block manager
adds a block where the new token starts one, or copies a shared last block.

Poisoning (correctness runs): free blocks, the slots after the last cached
token of each sequence, and table padding (-1) are filled with NaN (0x7F for
e4m3), so a kernel that reads a slot it must not read produces NaN.

Randomness: structure (lengths, free-list shuffle, stems) comes from
``numpy.random.default_rng(seed)``; values (pools, rows, queries) from a
``torch.Generator`` on the target device seeded with the same number, drawn
N(0, 1) in fp32 and rounded to the storage dtype.  The e4m3 pools use
``scale = amax / 448`` of the drawn fp32 data and torch's own e4m3 cast of
``x / scale`` (the values are inputs; the path's quantiser is the cache
write, which this module never performs).
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch

F32, F16, BF16, E4M3, E5M2 = "f32", "f16", "bf16", "e4m3", "e5m2"
TORCH_DTYPE = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16, E4M3: torch.uint8,
               E5M2: torch.uint8}
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2, E4M3: 1, E5M2: 1}
FP8_MAX = {E4M3: 448.0, E5M2: 57344.0}
FP8_TORCH = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


@dataclass(frozen=True)
class Config:
    name: str
    config_id: int
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    kv_dtype: str
    q_dtype: str
    out_dtype: str
    src_dtype: str              # dtype of the new K/V rows handed to the cache write
    lens: tuple = ()            # fixed lengths (tiny) ...
    len_range: tuple = ()       # ... or inclusive uniform range
    pool_blocks: int = 0        # fixed pool size, else needed * (1 + slack)
    slack: float = 0.10
    shared: dict = field(default_factory=dict)  # shared-prefix layout parameters
    partition_size: int = 512
    prefill: dict = field(default_factory=dict)  # prefill: inclusive ranges "new", "ctx"
    swap: dict = field(default_factory=dict)     # swap: blocks moved each way
    stream: dict = field(default_factory=dict)   # block-manager request stream parameters
    head_scales: bool = False   # 8-bit caches: one scale per KV head instead of one per pool

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def seed(self) -> int:
        return 412_000 + self.config_id


CONFIGS = {
    "tiny": Config("tiny", 1, B=4, Hq=8, Hkv=8, D=64, block_size=16, kv_dtype=F32, q_dtype=F32,
                   out_dtype=F32, src_dtype=F32, lens=(40, 17, 64, 1), pool_blocks=64),
    "llama13b": Config("llama13b", 2, B=64, Hq=40, Hkv=40, D=128, block_size=16, kv_dtype=F16,
                       q_dtype=F16, out_dtype=F16, src_dtype=F16, len_range=(128, 2048)),
    "llama70b": Config("llama70b", 3, B=256, Hq=64, Hkv=8, D=128, block_size=16, kv_dtype=BF16,
                       q_dtype=BF16, out_dtype=BF16, src_dtype=BF16, lens=(4096,) * 256),
    "shared": Config("shared", 4, B=96, Hq=40, Hkv=40, D=128, block_size=16, kv_dtype=F16,
                     q_dtype=F16, out_dtype=F16, src_dtype=F16,
                     shared=dict(prompts=32, samples=3, prefix=1024, stem=(64, 512))),
    "long_fp8": Config("long_fp8", 5, B=16, Hq=32, Hkv=8, D=128, block_size=16, kv_dtype=E4M3,
                       q_dtype=BF16, out_dtype=BF16, src_dtype=BF16, len_range=(16384, 32768)),
    "long_fp8_bs32": Config("long_fp8_bs32", 6, B=16, Hq=32, Hkv=8, D=128, block_size=32,
                            kv_dtype=E4M3, q_dtype=BF16, out_dtype=BF16, src_dtype=BF16,
                            len_range=(16384, 32768)),
    "long_fp8_heads": Config("long_fp8_heads", 13, B=16, Hq=32, Hkv=8, D=128, block_size=16,
                             kv_dtype=E4M3, q_dtype=BF16, out_dtype=BF16, src_dtype=BF16,
                             len_range=(16384, 32768), head_scales=True),
    "long_e5m2": Config("long_e5m2", 12, B=16, Hq=32, Hkv=8, D=128, block_size=16, kv_dtype=E5M2,
                        q_dtype=BF16, out_dtype=BF16, src_dtype=BF16, len_range=(16384, 32768)),
    # the 13B and 70B decode layers with other block sizes (8: a matrix-core
    # tile spans two blocks; 64: walked as 32-token halves)
    "llama13b_bs8": Config("llama13b_bs8", 14, B=64, Hq=40, Hkv=40, D=128, block_size=8,
                           kv_dtype=F16, q_dtype=F16, out_dtype=F16, src_dtype=F16,
                           len_range=(128, 2048)),
    "llama13b_bs64": Config("llama13b_bs64", 15, B=64, Hq=40, Hkv=40, D=128, block_size=64,
                            kv_dtype=F16, q_dtype=F16, out_dtype=F16, src_dtype=F16,
                            len_range=(128, 2048)),
    "llama70b_bs8": Config("llama70b_bs8", 16, B=256, Hq=64, Hkv=8, D=128, block_size=8,
                           kv_dtype=BF16, q_dtype=BF16, out_dtype=BF16, src_dtype=BF16,
                           lens=(4096,) * 256),
    "llama70b_bs64": Config("llama70b_bs64", 17, B=256, Hq=64, Hkv=8, D=128, block_size=64,
                            kv_dtype=BF16, q_dtype=BF16, out_dtype=BF16, src_dtype=BF16,
                            lens=(4096,) * 256),
    # prefill: several new tokens per sequence, causal over the paged context
    "prefill13b": Config("prefill13b", 7, B=16, Hq=40, Hkv=40, D=128, block_size=16, kv_dtype=F16,
                         q_dtype=F16, out_dtype=F16, src_dtype=F16,
                         prefill=dict(new=(512, 4096), ctx=(0, 0))),
    "prefill70b": Config("prefill70b", 8, B=16, Hq=64, Hkv=8, D=128, block_size=16, kv_dtype=BF16,
                         q_dtype=BF16, out_dtype=BF16, src_dtype=BF16,
                         prefill=dict(new=(1024, 1024), ctx=(0, 3072))),
    "prefill70b_bs8": Config("prefill70b_bs8", 18, B=16, Hq=64, Hkv=8, D=128, block_size=8,
                             kv_dtype=BF16, q_dtype=BF16, out_dtype=BF16, src_dtype=BF16,
                             prefill=dict(new=(1024, 1024), ctx=(0, 3072))),
    "prefill70b_bs64": Config("prefill70b_bs64", 19, B=16, Hq=64, Hkv=8, D=128, block_size=64,
                              kv_dtype=BF16, q_dtype=BF16, out_dtype=BF16, src_dtype=BF16,
                              prefill=dict(new=(1024, 1024), ctx=(0, 3072))),
    "prefill_fp8": Config("prefill_fp8", 9, B=8, Hq=32, Hkv=8, D=128, block_size=16, kv_dtype=E4M3,
                          q_dtype=BF16, out_dtype=BF16, src_dtype=BF16,
                          prefill=dict(new=(2048, 2048), ctx=(0, 6144))),
    # host block manager: continuous batching over shared system prompts
    "prefix_stream": Config("prefix_stream", 11, B=256, Hq=40, Hkv=40, D=128, block_size=16,
                            kv_dtype=F16, q_dtype=F16, out_dtype=F16, src_dtype=F16,
                            stream=dict(requests=3000, systems=8, system_len=(256, 2048),
                                        user_len=(16, 256), gen_len=(32, 256), p_system=0.8,
                                        p_samples=0.25, samples=3)),
    # page-granular eviction to pinned host memory and restore (13B block shape)
    "swap13b": Config("swap13b", 10, B=0, Hq=40, Hkv=40, D=128, block_size=16, kv_dtype=F16,
                      q_dtype=F16, out_dtype=F16, src_dtype=F16, swap=dict(blocks=1024)),
}


def small(cfg: Config, **kw) -> Config:
    """A reduced copy of a config for oracle-speed parity runs."""
    return replace(cfg, **kw)


@dataclass
class Workload:
    """Pre-step state of one decode step plus the new token's rows.

    Host-side structure (NumPy): ``seq_lens`` (L, including the new token),
    ``tables`` (list of lists: pre-step block tables), ``refs`` (block ->
    number of tables that reference it), ``free`` (remaining free list, FIFO
    order).  Device tensors: ``q [B,Hq,D]``, ``k_pool``/``v_pool``
    ``[NB,bs,Hkv,D]``, ``k_new``/``v_new`` ``[B,Hkv,D]``.
    """

    cfg: Config
    seq_lens: np.ndarray
    tables: list
    refs: dict
    free: list
    num_blocks: int
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    k_scale: float = 1.0
    v_scale: float = 1.0
    scale: float = 0.0

    @property
    def max_blocks(self) -> int:
        bs = self.cfg.block_size
        return max(1, max(-(-int(L) // bs) for L in self.seq_lens))


def _ceil_div(a: int, b: int) -> int:
    return -(-int(a) // int(b))


def _poison_value(dtype: str):
    return 0x7F if dtype in FP8_MAX else float("nan")


def _fill_values(shape, dtype: str, gen: torch.Generator, device, sigma: float = 1.0,
                 per_head: bool = False):
    """N(0, sigma^2) draws rounded to ``dtype``; 8-bit formats return (codes,
    scale) with scale = amax / (the format's largest finite value).  With
    ``per_head`` (8-bit pools [NB, bs, Hkv, D]) each KV head's draws are first
    multiplied by 2^u, u uniform in [-4, 4], and the scale is a float32 array
    with one amax-based scale per head."""
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    if dtype in FP8_MAX and per_head:
        H = shape[2]
        mag = torch.exp2(torch.rand(H, generator=gen, device=device) * 8.0 - 4.0)
        x.mul_(mag.view(1, 1, H, 1))
        amax = x.abs().amax(dim=(0, 1, 3))
        scale = (amax / FP8_MAX[dtype]).to(torch.float32)
        codes = (x / scale.view(1, 1, H, 1)).clamp_(-FP8_MAX[dtype], FP8_MAX[dtype])
        return codes.to(FP8_TORCH[dtype]).view(torch.uint8), scale.cpu().numpy()
    if dtype in FP8_MAX:
        scale = float(x.abs().max()) / FP8_MAX[dtype]
        codes = (x / scale).clamp_(-FP8_MAX[dtype], FP8_MAX[dtype]).to(FP8_TORCH[dtype]).view(torch.uint8)
        return codes, scale
    return x.to(TORCH_DTYPE[dtype]), 1.0


def _lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.lens:
        return np.array(cfg.lens[: cfg.B], dtype=np.int64)
    lo, hi = cfg.len_range
    return rng.integers(lo, hi, size=cfg.B, endpoint=True).astype(np.int64)


def seq_lengths(cfg: Config) -> np.ndarray:
    """The lengths (new token included) ``make`` gives the sequences of
    ``cfg``: the first draws of the config's generator."""
    rng = np.random.default_rng(cfg.seed)
    if cfg.shared:
        sh = cfg.shared
        stems = rng.integers(sh["stem"][0], sh["stem"][1], size=sh["prompts"], endpoint=True)
        return np.repeat(sh["prefix"] + stems.astype(np.int64) + 1, sh["samples"])
    return _lengths(cfg, rng)


def make(cfg: Config, device="cpu", poison: bool = True, q_sigma: float = 1.0) -> Workload:
    """Build the seeded pre-step state of ``cfg`` on ``device``."""
    if cfg.shared:
        return _make_shared(cfg, device, poison, q_sigma)
    rng = np.random.default_rng(cfg.seed)
    gen = torch.Generator(device=device).manual_seed(cfg.seed)
    bs = cfg.block_size
    lens = _lengths(cfg, rng)
    cached = np.maximum(lens - 1, 0)                 # tokens already in the cache
    need_total = int(sum(_ceil_div(L, bs) for L in lens))
    NB = cfg.pool_blocks or int(np.ceil(need_total * (1.0 + cfg.slack)))
    if NB < need_total:
        raise ValueError("pool too small")
    free = [int(b) for b in rng.permutation(NB)]
    tables, refs = [], {}
    for c in cached:
        row = [free.pop(0) for _ in range(_ceil_div(int(c), bs))]
        for blk in row:
            refs[blk] = 1
        tables.append(row)
    wl = _values(cfg, device, gen, lens, tables, NB, free, refs, poison, q_sigma)
    return wl


def _make_shared(cfg: Config, device, poison: bool, q_sigma: float) -> Workload:
    sh = cfg.shared
    rng = np.random.default_rng(cfg.seed)
    gen = torch.Generator(device=device).manual_seed(cfg.seed)
    bs = cfg.block_size
    P, S, prefix = sh["prompts"], sh["samples"], sh["prefix"]
    stems = rng.integers(sh["stem"][0], sh["stem"][1], size=P, endpoint=True).astype(np.int64)
    lens = np.repeat(prefix + stems + 1, S)           # L includes the new token
    # blocks: prefix + stems + one possible new/copied block per sample
    need_shared = _ceil_div(prefix, bs) + int(sum(_ceil_div(int(c), bs) for c in stems))
    NB = int(np.ceil((need_shared + P * S) * (1.0 + cfg.slack)))
    free = [int(b) for b in rng.permutation(NB)]
    refs = {}
    prefix_row = [free.pop(0) for _ in range(_ceil_div(prefix, bs))]
    if prefix % bs:
        raise ValueError("the shared prefix is assumed to fill whole blocks")
    for blk in prefix_row:
        refs[blk] = P * S
    tables = []
    for p in range(P):
        stem_row = [free.pop(0) for _ in range(_ceil_div(int(stems[p]), bs))]
        for blk in stem_row:
            refs[blk] = S
        for _ in range(S):
            tables.append(prefix_row + stem_row)
    return _values(cfg, device, gen, lens, tables, NB, free, refs, poison, q_sigma)


def _values(cfg, device, gen, lens, tables, NB, free, refs, poison, q_sigma) -> Workload:
    bs, Hkv, D = cfg.block_size, cfg.Hkv, cfg.D
    k_pool, k_scale = _fill_values((NB, bs, Hkv, D), cfg.kv_dtype, gen, device, per_head=cfg.head_scales)
    v_pool, v_scale = _fill_values((NB, bs, Hkv, D), cfg.kv_dtype, gen, device, per_head=cfg.head_scales)
    if poison:
        pv = _poison_value(cfg.kv_dtype)
        used = np.zeros(NB, dtype=bool)
        for row in tables:
            used[row] = True
        free_ids = torch.as_tensor(np.nonzero(~used)[0], device=device, dtype=torch.long)
        k_pool.index_fill_(0, free_ids, pv)
        v_pool.index_fill_(0, free_ids, pv)
        # slots after the last cached token of each distinct table
        seen = set()
        for row, L in zip(tables, lens):
            cached = max(int(L) - 1, 0)
            if not row or cached % bs == 0:
                continue
            key = (row[-1], cached % bs)
            if key in seen:
                continue
            seen.add(key)
            k_pool[row[-1], cached % bs:] = pv
            v_pool[row[-1], cached % bs:] = pv
    B, Hq = cfg.B, cfg.Hq
    k_new, _ = _fill_values((B, Hkv, D), cfg.src_dtype, gen, device)
    v_new, _ = _fill_values((B, Hkv, D), cfg.src_dtype, gen, device)
    q, _ = _fill_values((B, Hq, D), cfg.q_dtype, gen, device, sigma=q_sigma)
    return Workload(cfg=cfg, seq_lens=np.asarray(lens, dtype=np.int64), tables=tables, refs=refs,
                    free=free, num_blocks=NB, q=q, k_pool=k_pool, v_pool=v_pool, k_new=k_new,
                    v_new=v_new, k_scale=k_scale, v_scale=v_scale, scale=1.0 / float(np.sqrt(D)))


def pad_tables(tables: list, width: int) -> np.ndarray:
    """Rows of block ids padded with -1 to ``width`` (int32)."""
    out = np.full((len(tables), width), -1, dtype=np.int32)
    for i, row in enumerate(tables):
        out[i, : len(row)] = row
    return out


@dataclass
class PrefillWorkload:
    """State before one prefill call plus the new tokens' rows.

    Sequence b holds ``ctx[b]`` cached tokens and receives ``news[b]`` new
    ones, so ``seq_lens[b] = ctx[b] + news[b]``; its table already lists the
    ceil(seq_lens[b] / bs) blocks of all of them (allocated FIFO from the
    shuffled free list).  Device tensors: ``q [T,Hq,D]`` and ``k_new``/
    ``v_new [T,Hkv,D]`` packed by sequence (``q_starts``), pools
    ``[NB,bs,Hkv,D]`` holding the cached tokens.
    """

    cfg: Config
    seq_lens: np.ndarray
    news: np.ndarray
    q_starts: np.ndarray
    tables: list
    num_blocks: int
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    k_scale: float = 1.0
    v_scale: float = 1.0
    scale: float = 0.0

    @property
    def T(self) -> int:
        return int(self.q_starts[-1])

    @property
    def max_blocks(self) -> int:
        bs = self.cfg.block_size
        return max(1, max(-(-int(L) // bs) for L in self.seq_lens))


def prefill_lengths(cfg: Config):
    """(new tokens, cached tokens) per sequence: the first draws of the
    config's generator, new counts first."""
    rng = np.random.default_rng(cfg.seed)
    lo, hi = cfg.prefill["new"]
    news = rng.integers(lo, hi, size=cfg.B, endpoint=True).astype(np.int64)
    lo, hi = cfg.prefill["ctx"]
    ctx = rng.integers(lo, hi, size=cfg.B, endpoint=True).astype(np.int64)
    return news, ctx, rng


def make_prefill(cfg: Config, device="cpu", poison: bool = True, lengths=None) -> PrefillWorkload:
    """Build the seeded pre-prefill state of ``cfg`` on ``device``.

    Draw order: new counts, cached counts, free-list shuffle, then values
    (K pool, V pool, new K rows, new V rows, q).  ``lengths`` = (news, ctx)
    replaces the drawn counts (edge-case tests).  With ``poison`` the free
    blocks, the new tokens' slots (the cache write fills them) and the slots
    past each sequence's end are NaN (0x7F for e4m3)."""
    news, ctx, rng = prefill_lengths(cfg)
    if lengths is not None:
        news = np.asarray(lengths[0], dtype=np.int64)
        ctx = np.asarray(lengths[1], dtype=np.int64)
        if len(news) != cfg.B or len(ctx) != cfg.B:
            raise ValueError("lengths must give B entries each")
    gen = torch.Generator(device=device).manual_seed(cfg.seed)
    bs, Hkv, D, Hq = cfg.block_size, cfg.Hkv, cfg.D, cfg.Hq
    lens = ctx + news
    need = int(sum(_ceil_div(int(L), bs) for L in lens))
    NB = cfg.pool_blocks or int(np.ceil(need * (1.0 + cfg.slack)))
    free = [int(b) for b in rng.permutation(NB)]
    tables = [[free.pop(0) for _ in range(_ceil_div(int(L), bs))] for L in lens]
    k_pool, k_scale = _fill_values((NB, bs, Hkv, D), cfg.kv_dtype, gen, device, per_head=cfg.head_scales)
    v_pool, v_scale = _fill_values((NB, bs, Hkv, D), cfg.kv_dtype, gen, device, per_head=cfg.head_scales)
    if poison:
        pv = _poison_value(cfg.kv_dtype)
        used = np.zeros(NB, dtype=bool)
        for row in tables:
            used[row] = True
        free_ids = torch.as_tensor(np.nonzero(~used)[0], device=device, dtype=torch.long)
        k_pool.index_fill_(0, free_ids, pv)
        v_pool.index_fill_(0, free_ids, pv)
        for row, c in zip(tables, ctx):
            c = int(c)
            for j in range(c // bs, len(row)):   # blocks holding new tokens or nothing
                first = c % bs if j == c // bs else 0
                k_pool[row[j], first:] = pv
                v_pool[row[j], first:] = pv
    starts = np.concatenate([[0], np.cumsum(news)]).astype(np.int64)
    T = int(starts[-1])
    k_new, _ = _fill_values((T, Hkv, D), cfg.src_dtype, gen, device)
    v_new, _ = _fill_values((T, Hkv, D), cfg.src_dtype, gen, device)
    q, _ = _fill_values((T, Hq, D), cfg.q_dtype, gen, device)
    return PrefillWorkload(cfg=cfg, seq_lens=lens, news=news, q_starts=starts, tables=tables,
                           num_blocks=NB, q=q, k_pool=k_pool, v_pool=v_pool, k_new=k_new,
                           v_new=v_new, k_scale=k_scale, v_scale=v_scale,
                           scale=1.0 / float(np.sqrt(D)))


@dataclass
class SwapWorkload:
    """Device pools, pinned host pools and the two block mappings of one
    eviction and restore: ``out_map`` (device block -> host block) and
    ``in_map`` (host block -> another device block), int32 [N, 2] on the GPU."""

    cfg: Config
    k_dev: torch.Tensor
    v_dev: torch.Tensor
    k_host: torch.Tensor
    v_host: torch.Tensor
    out_pairs: np.ndarray
    in_pairs: np.ndarray
    out_map: torch.Tensor
    in_map: torch.Tensor

    @property
    def block_bytes(self) -> int:
        c = self.cfg
        return c.block_size * c.Hkv * c.D * ELEM_BYTES[c.kv_dtype]


def make_swap(cfg: Config, device="cuda") -> SwapWorkload:
    """A device pool of 2N + N/8 blocks, N of them (a seeded random choice)
    evicted to host blocks 0..N-1 and restored to N other device blocks."""
    N = int(cfg.swap["blocks"])
    rng = np.random.default_rng(cfg.seed)
    NB = 2 * N + N // 8
    perm = rng.permutation(NB)
    victims, targets = perm[:N], perm[N:2 * N]
    gen = torch.Generator(device=device).manual_seed(cfg.seed)
    k_dev, _ = _fill_values((NB, cfg.block_size, cfg.Hkv, cfg.D), cfg.kv_dtype, gen, device)
    v_dev, _ = _fill_values((NB, cfg.block_size, cfg.Hkv, cfg.D), cfg.kv_dtype, gen, device)
    shape = (N, cfg.block_size, cfg.Hkv, cfg.D)
    k_host = torch.zeros(shape, dtype=k_dev.dtype).pin_memory()
    v_host = torch.zeros(shape, dtype=v_dev.dtype).pin_memory()
    host_ids = rng.permutation(N)
    out_pairs = np.stack([victims, host_ids], axis=1).astype(np.int32)
    in_pairs = np.stack([host_ids, targets], axis=1).astype(np.int32)
    return SwapWorkload(cfg, k_dev, v_dev, k_host, v_host, out_pairs, in_pairs,
                        torch.from_numpy(out_pairs).to(device), torch.from_numpy(in_pairs).to(device))


def make_stream(cfg: Config) -> list:
    """The operation trace of ``cfg``'s request stream, as a list of
    ("add", tokens) / ("append", seq, token) / ("fork", seq) / ("free", seq)
    tuples.  Sequence ids are the order of creation (adds and forks), as the
    block manager numbers them.  Each decode step appends one token to every
    live sequence; finished sequences are freed; new requests fill the
    batch up to ``cfg.B`` sequences."""
    p = cfg.stream
    rng = np.random.default_rng(cfg.seed)
    systems = [rng.integers(0, 32000, size=int(rng.integers(p["system_len"][0], p["system_len"][1],
                                                          endpoint=True))).tolist()
               for _ in range(p["systems"])]
    ops, live, next_id, admitted = [], {}, 0, 0
    while admitted < p["requests"] or live:
        while admitted < p["requests"] and len(live) + p["samples"] <= cfg.B:
            prompt = (systems[int(rng.integers(p["systems"]))] if rng.random() < p["p_system"] else [])
            user = rng.integers(0, 32000, size=int(rng.integers(p["user_len"][0], p["user_len"][1],
                                                                endpoint=True))).tolist()
            ops.append(("add", prompt + user))
            first = next_id
            next_id += 1
            live[first] = int(rng.integers(p["gen_len"][0], p["gen_len"][1], endpoint=True))
            if rng.random() < p["p_samples"]:
                for _ in range(p["samples"] - 1):
                    ops.append(("fork", first))
                    live[next_id] = int(rng.integers(p["gen_len"][0], p["gen_len"][1], endpoint=True))
                    next_id += 1
            admitted += 1
        for sid in list(live):
            ops.append(("append", sid, int(rng.integers(0, 32000))))
            live[sid] -= 1
            if live[sid] == 0:
                ops.append(("free", sid))
                del live[sid]
    return ops


def scale_args(wl, device):
    """(k_scale, v_scale, k_scales, v_scales) for the library: pool-wide
    floats, or per-head device tensors with the floats left at 1."""
    if isinstance(wl.k_scale, np.ndarray):
        ks = torch.from_numpy(np.ascontiguousarray(wl.k_scale, dtype=np.float32)).to(device)
        vs = torch.from_numpy(np.ascontiguousarray(wl.v_scale, dtype=np.float32)).to(device)
        return 1.0, 1.0, ks, vs
    return wl.k_scale, wl.v_scale, None, None
