"""One decode step of the paged KV cache on the GPU, through the C ABI.

A step, for a batch whose caches hold L-1 tokens each:

1. the host block manager gives every sequence room for its new token (a new
   block when the last one is full, a copy-on-write when the last block is
   shared) -- done once, when the step is prepared;
2. ``pa_copy_blocks``      copy-on-write block copies (when there are any);
3. ``pa_append_kv``        slot of each new token from the block tables and
   the write of its K/V rows there, in one launch (equal to
   ``pa_slot_mapping`` followed by ``pa_reshape_and_cache``);
4. ``pa_decode_partition`` paged attention (sequences split across
   work-groups combined in the same launch, or:)
5. ``pa_decode_reduce``    the reduce launch that combines them, when the
   library combines them in a launch of its own.

Steps 2-5 run on the GPU and are what :meth:`DecodeStep.run` enqueues; they
are idempotent, so the same prepared step can be replayed for timing.
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding
from .blocks import BlockManager
from .workloads import TORCH_DTYPE, Workload, pad_tables, scale_args


class DecodeStep:
    def __init__(self, wl: Workload, partition_size: int = 0, out_dtype=None, device="cuda",
                 combine=binding.PA_COMBINE_AUTO):
        cfg = wl.cfg
        self.wl = wl
        bs = cfg.block_size
        mgr = BlockManager(wl.num_blocks, bs, free=wl.free, refs=wl.refs)
        self.tables_list, self.copies = mgr.plan_step(wl.tables, wl.seq_lens - 1)
        width = max(1, max(len(r) for r in self.tables_list))
        self.tables_np = pad_tables(self.tables_list, width)
        dev = torch.device(device)
        self.block_tables = torch.from_numpy(self.tables_np).to(dev)
        self.seq_lens = torch.from_numpy(wl.seq_lens.astype(np.int32)).to(dev)
        pos = np.where(wl.seq_lens > 0, wl.seq_lens - 1, -1).astype(np.int32)
        self.positions = torch.from_numpy(pos).to(dev)
        self.slots = torch.empty(cfg.B, dtype=torch.int32, device=dev)
        self.mapping = (torch.tensor(self.copies, dtype=torch.int32, device=dev).reshape(-1, 2)
                        if self.copies else torch.empty((0, 2), dtype=torch.int32, device=dev))
        odt = out_dtype or cfg.out_dtype
        self.out = torch.empty((cfg.B, cfg.Hq, cfg.D), dtype=TORCH_DTYPE[odt], device=dev)
        self.kv_dtype = cfg.kv_dtype
        self.k_scale, self.v_scale, self.k_scales, self.v_scales = scale_args(wl, dev)
        self.args = binding.decode_args(self.out, wl.q, wl.k_pool, wl.v_pool, self.block_tables,
                                        self.seq_lens, wl.scale, self.k_scale, self.v_scale,
                                        partition_size, None, cfg.kv_dtype, self.k_scales,
                                        self.v_scales, combine)
        self.workspace = binding.alloc_workspace(self.args, dev)

    # individual stages (each one C-ABI call)
    def slot_mapping(self, stream=None):
        binding.slot_mapping(self.block_tables, self.positions, self.wl.cfg.block_size, self.slots, stream)

    def copy_blocks(self, stream=None):
        if self.mapping.shape[0]:
            binding.copy_blocks(self.wl.k_pool, self.wl.v_pool, self.mapping, self.kv_dtype, stream)

    def cache_write(self, stream=None):
        wl = self.wl
        binding.reshape_and_cache(wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, self.slots, self.k_scale,
                                  self.v_scale, self.kv_dtype, stream, self.k_scales, self.v_scales)

    def append_kv(self, stream=None):
        """Slot mapping and cache write in one launch (pa_append_kv)."""
        wl = self.wl
        binding.append_kv(wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, self.block_tables, self.positions,
                          self.slots, self.k_scale, self.v_scale, self.kv_dtype, stream, self.k_scales,
                          self.v_scales)

    def decode_partition(self, stream=None):
        binding.decode_partition_run(self.args, stream)

    def decode_reduce(self, stream=None):
        binding.decode_reduce_run(self.args, stream)

    # the step: copy-on-write copies first (the new token may land in a
    # copied block), then the new token's slot and K/V rows, attention, reduce
    STAGES = ("copy_blocks", "append_kv", "decode_partition", "decode_reduce")

    def run(self, stream=None):
        for s in self.STAGES:
            getattr(self, s)(stream)
        return self.out

    def run_unfused(self, stream=None):
        """The same step with the slot mapping and the cache write as two calls."""
        self.slot_mapping(stream)
        self.copy_blocks(stream)
        self.cache_write(stream)
        self.decode_partition(stream)
        self.decode_reduce(stream)
        return self.out


class PrefillStep:
    """One prefill call of the paged KV cache on the GPU, through the C ABI.

    The sequences' tables already hold blocks for every new token (the host
    block manager allocates them when the prompt is admitted).  A call:

    1. ``pa_prefill_slot_mapping`` slot of every new token;
    2. ``pa_reshape_and_cache``    write the new K/V rows to their slots;
    3. ``pa_prefill``              causal paged attention of the new tokens.

    All three are idempotent, so the prepared call can be replayed for timing.
    """

    def __init__(self, wl, out_dtype=None, device="cuda"):
        cfg = wl.cfg
        self.wl = wl
        dev = torch.device(device)
        width = max(1, max(len(r) for r in wl.tables))
        self.tables_np = pad_tables(wl.tables, width)
        self.block_tables = torch.from_numpy(self.tables_np).to(dev)
        self.seq_lens = torch.from_numpy(wl.seq_lens.astype(np.int32)).to(dev)
        self.q_starts = torch.from_numpy(wl.q_starts.astype(np.int32)).to(dev)
        self.max_q_len = int(max(wl.news)) if len(wl.news) else 0
        self.slots = torch.empty(wl.T, dtype=torch.int32, device=dev)
        odt = out_dtype or cfg.out_dtype
        self.out = torch.empty((wl.T, cfg.Hq, cfg.D), dtype=TORCH_DTYPE[odt], device=dev)
        self.kv_dtype = cfg.kv_dtype
        self.k_scale, self.v_scale, self.k_scales, self.v_scales = scale_args(wl, dev)
        self.args = binding.prefill_args(self.out, wl.q, wl.k_pool, wl.v_pool, self.block_tables,
                                         self.seq_lens, self.q_starts, self.max_q_len, wl.scale,
                                         self.k_scale, self.v_scale, cfg.kv_dtype, self.k_scales,
                                         self.v_scales)

    def slot_mapping(self, stream=None):
        binding.prefill_slot_mapping(self.block_tables, self.seq_lens, self.q_starts,
                                     self.wl.cfg.block_size, self.slots, stream)

    def cache_write(self, stream=None):
        wl = self.wl
        binding.reshape_and_cache(wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, self.slots, self.k_scale,
                                  self.v_scale, self.kv_dtype, stream, self.k_scales, self.v_scales)

    def attention(self, stream=None):
        binding.prefill_run(self.args, stream)

    def run(self, stream=None):
        self.slot_mapping(stream)
        self.cache_write(stream)
        self.attention(stream)
        return self.out
