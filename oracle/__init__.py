"""CPU oracle for the paged KV-cache decode path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
restatement of what the paged decode path computes, in NumPy float64.  Only the
test suite, the smoke check in ``__graft_entry__`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The GPU library and its Python binding
never import, call or link anything here, and nothing here imports them: the
two sides share no kernels, headers, helpers, tables or constants.

Sources (three web pages on PagedAttention, cited by title and section):

* P1 -- Ultralytics glossary page "PagedAttention" (Turkish).  Sections:
  the introduction; "Çözdüğü Bellek Sorunu" (the memory problem it solves);
  "Sayfalama Nasıl Çalışır" (how paging works -- prose, a PyTorch code
  sketch of a block pool, a free list and a block table, and the output the
  sketch prints); "Diziler Arasında Blokları Paylaşma" (sharing blocks
  between sequences); "İlgili Teknikler" (related techniques: FlashAttention,
  continuous batching, grouped-query attention, FP8 cache quantisation).
* P2 -- infolopare.com news item "PagedAttention: Unapređivanje propusnosti
  sistema za usluživanje jezičkih modela velikih razmera" (Serbian), one
  section.
* P3 -- gyaansetu.com page "حافظه KV و PagedAttention: چرا سرور LLM شما کند
  میشود؟" (KV memory and PagedAttention: why is your LLM server slow?),
  Persian, two articles: A (sections "مشکل حافظه" the memory problem, "چگونه
  PagedAttention این مشکل را حل میکند" how it solves it) and B "KV Cache و
  PagedAttention" (sections "KV Cache چیست؟" what the KV cache is, "مشکل
  کجاست؟" internal and external fragmentation, "راه حل: PagedAttention" the
  solution, "مزایای PagedAttention" benefits).

Modules:

* :mod:`oracle.numerics` -- bit-level decoding of fp32/fp16/bf16 storage to
  float64 and correctly rounded encoding to binary floating-point formats.
* :mod:`oracle.fp8` -- the OCP e4m3 ("fn") codec, written from the format's
  definition; the encoder rounds to nearest-even and saturates.
* :mod:`oracle.paged` -- slot mapping, the cache write, the block copy, the
  gather through the block table and float64 softmax attention: decode (one
  new token per sequence) and prefill (several new tokens per sequence,
  causal).
* :mod:`oracle.blocks` -- the host-side block bookkeeping the pages describe:
  FIFO free list, per-block reference counts, allocation of a new block only
  when the last one is full, and copy-on-write of shared blocks.
* :mod:`oracle.prefix_cache` -- the host block manager with content-hashed
  prefix caching (FNV-1a keys over whole prefixes), LRU reuse of released
  cached blocks and free-on-finish.
* :mod:`oracle.sizes` -- the KV-cache size and waste arithmetic the pages
  quote.

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (worked example, closed forms, library special cases, brute force,
invariants) except where its docstring says "parity unpinned".
"""

from . import numerics, fp8, paged, blocks, prefix_cache, sizes  # noqa: F401
