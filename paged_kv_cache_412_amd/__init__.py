"""Paged KV-cache decode path for AMD Instinct MI355X (gfx950).

The compute lives in ``libpa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/pa.h``).  :mod:`paged_kv_cache_412_amd.binding` marshals
torch tensors into that ABI; :mod:`paged_kv_cache_412_amd.blocks` is the host
block manager (free list, reference counts, copy-on-write planning);
:mod:`paged_kv_cache_412_amd.workloads` makes seeded synthetic inputs.
"""
