"""KV-cache size and waste arithmetic (test infrastructure only).

The pages quote cache sizes and waste figures; these closed forms reproduce
them and fix the bytes-per-token formula that the throughput metric counts.

* A transformer keeps one key and one value vector per token in every layer
  (P1 "Çözdüğü Bellek Sorunu"; P3 article B "KV Cache چیست؟"), so one token
  costs ``2 * layers * Hkv * D * elem_bytes`` bytes.
* Paged storage wastes only the unfilled part of each sequence's last block
  (P1 "Sayfalama Nasıl Çalışır"); a contiguous reservation wastes everything
  past the tokens used (P1 "Çözdüğü Bellek Sorunu"; P3 article A, internal
  fragmentation; P3 article B "مشکل کجاست؟").

Pinned by the figures the pages print: LLaMA-13B up to 1.7 GB per sequence,
Llama-3.1-70B about 1.3 GB per 4,096-token sequence and 336 GB for 256 users,
93 % waste for 300 of 4,096, 950 of 1,000 unused, 8 vs 2,008 unused slots.
"""

from __future__ import annotations


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V, every layer: 2 * layers * Hkv * D * elem_bytes."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


def kv_bytes(tokens: int, layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return tokens * kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes)


def paged_unused_slots(length: int, block_size: int) -> int:
    """Unfilled slots of the last block: ceil(L/bs)*bs - L."""
    return -(-length // block_size) * block_size - length


def reserved_unused_slots(length: int, reservation: int) -> int:
    """Slots a contiguous max-length reservation leaves unused."""
    return reservation - length


def waste_fraction(used: int, reserved: int) -> float:
    return 1.0 - used / reserved
