// pa_block_manager.cpp -- the host block manager of libpa: which physical
// block each sequence's table points at, with content-hashed prefix caching
// across requests.  Host code only; declarations in include/pa.h.
//
// P1 = Ultralytics glossary page "PagedAttention".
//  * FIFO free list: blocks leave from the front and return to the back
//    ("Sayfalama Nasıl Çalışır": the code sketch pops free ids from the
//    front of a list).
//  * A new block only when the last one is full (same section; P3 article A,
//    on-demand allocation).
//  * Reference counts and copy-on-write of shared blocks ("Diziler Arasında
//    Blokları Paylaşma"; P3 article A, shared prefixes).
//  * Hashing every block to share cached blocks across requests that start
//    with the same tokens (P1 "Diziler Arasında Blokları Paylaşma", prompt
//    caching), and returning a finished sequence's blocks at once ("İlgili
//    Teknikler", continuous batching).
//
// Keys: a full block's key is the 64-bit FNV-1a hash of every token from
// the start of the sequence through the end of the block (token ids as
// 4-byte little-endian integers), computed incrementally: each block's key
// continues its parent's.  A hit also compares the block's stored tokens and
// parent key, so a hash collision never shares a block.  Released blocks with
// a key stay cached on an LRU list until a new block is needed and the free
// list is empty.

#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

uint64_t fnv1a(uint64_t h, const int32_t* t, int n) {
  for (int i = 0; i < n; ++i) {
    const uint32_t v = static_cast<uint32_t>(t[i]);
    for (int k = 0; k < 4; ++k) {
      h ^= (v >> (8 * k)) & 0xffu;
      h *= kFnvPrime;
    }
  }
  return h;
}

struct Seq {
  std::vector<int32_t> tokens;
  std::vector<int32_t> table;
  std::vector<uint64_t> keys;  // keys of the full blocks so far
};

}  // namespace

struct pa_block_manager {
  int32_t nb = 0, bs = 0;
  bool caching = true;
  std::deque<int32_t> free;
  // evictable blocks: intrusive list, oldest release at the head
  std::vector<int32_t> prev, next;
  int32_t head = -1, tail = -1, n_evict = 0;
  std::vector<int32_t> refs;
  std::vector<uint8_t> keyed, in_evict;
  std::vector<uint64_t> key, parent;
  std::vector<int32_t> block_tokens;  // nb * bs: tokens of keyed blocks
  std::unordered_map<uint64_t, int32_t> owner;
  std::unordered_map<int32_t, Seq> seqs;
  int32_t next_id = 0;

  int32_t available() const { return static_cast<int32_t>(free.size()) + n_evict; }

  void evict_push(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in_evict[b] = 1;
    ++n_evict;
  }
  void evict_remove(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    in_evict[b] = 0;
    --n_evict;
  }

  // a new block for one user: the free list first, then the longest-released
  // cached block (which loses its key); the caller checked availability
  int32_t take() {
    int32_t b;
    if (!free.empty()) {
      b = free.front();
      free.pop_front();
    } else {
      b = head;
      evict_remove(b);
      owner.erase(key[b]);
      keyed[b] = 0;
    }
    refs[b] = 1;
    return b;
  }

  void release(int32_t b) {
    if (--refs[b] == 0) {
      if (keyed[b]) evict_push(b); else free.push_back(b);
    }
  }

  int32_t lookup(uint64_t k, uint64_t par, const int32_t* toks) const {
    auto it = owner.find(k);
    if (it == owner.end()) return -1;
    const int32_t b = it->second;
    if (parent[b] != par) return -1;
    const int32_t* have = &block_tokens[static_cast<size_t>(b) * bs];
    for (int i = 0; i < bs; ++i)
      if (have[i] != toks[i]) return -1;
    return b;
  }

  void register_key(int32_t b, uint64_t k, uint64_t par, const int32_t* toks) {
    if (!caching || keyed[b] || owner.count(k)) return;
    keyed[b] = 1;
    key[b] = k;
    parent[b] = par;
    owner.emplace(k, b);
    int32_t* dst = &block_tokens[static_cast<size_t>(b) * bs];
    for (int i = 0; i < bs; ++i) dst[i] = toks[i];
  }
};

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t prefix_caching,
                               const int32_t* free_order) {
  if (num_blocks < 1 || block_size < 1) return nullptr;
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX) return nullptr;
  pa_block_manager* m = new (std::nothrow) pa_block_manager();
  if (!m) return nullptr;
  try {
    m->nb = num_blocks;
    m->bs = block_size;
    m->caching = prefix_caching != 0;
    m->prev.assign(num_blocks, -1);
    m->next.assign(num_blocks, -1);
    m->refs.assign(num_blocks, 0);
    m->keyed.assign(num_blocks, 0);
    m->in_evict.assign(num_blocks, 0);
    m->key.assign(num_blocks, 0);
    m->parent.assign(num_blocks, 0);
    if (m->caching) m->block_tokens.assign(static_cast<size_t>(num_blocks) * block_size, 0);
    std::vector<uint8_t> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order ? free_order[i] : i;
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete m;
        return nullptr;  // not a permutation of the pool
      }
      seen[b] = 1;
      m->free.push_back(b);
    }
  } catch (...) {
    delete m;
    return nullptr;
  }
  return m;
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

pa_status pa_bm_add(pa_block_manager* m, const int32_t* tokens, int32_t n, int32_t* seq,
                    int32_t* cached_tokens) {
  if (!m || !seq || !cached_tokens || (n > 0 && !tokens)) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  const int bs = m->bs;
  const int nfull = n / bs;
  const int nblocks = (n + bs - 1) / bs;
  std::vector<uint64_t> keys, parents;
  int hits = 0, revived = 0;
  if (m->caching) {
    keys.resize(nfull);
    parents.resize(nfull);
    uint64_t h = kFnvOffset;
    for (int j = 0; j < nfull; ++j) {
      parents[j] = h;
      h = fnv1a(h, tokens + static_cast<size_t>(j) * bs, bs);
      keys[j] = h;
    }
    for (int j = 0; j < nfull; ++j) {
      const int32_t b = m->lookup(keys[j], parents[j], tokens + static_cast<size_t>(j) * bs);
      if (b < 0) break;
      ++hits;
      if (m->refs[b] == 0) ++revived;
    }
  }
  if (nblocks - hits > m->available() - revived) return PA_ERR_OUT_OF_BLOCKS;
  Seq s;
  s.tokens.assign(tokens, tokens + n);
  s.table.reserve(nblocks);
  for (int j = 0; j < hits; ++j) {
    const int32_t b = m->owner.find(keys[j])->second;
    if (m->refs[b] == 0) {
      m->evict_remove(b);
      m->refs[b] = 1;
    } else {
      ++m->refs[b];
    }
    s.table.push_back(b);
  }
  for (int j = hits; j < nblocks; ++j) {
    const int32_t b = m->take();
    s.table.push_back(b);
    if (j < nfull && m->caching)
      m->register_key(b, keys[j], parents[j], tokens + static_cast<size_t>(j) * bs);
  }
  s.keys = std::move(keys);
  const int32_t id = m->next_id++;
  m->seqs.emplace(id, std::move(s));
  *seq = id;
  *cached_tokens = hits * bs;
  return PA_OK;
}

pa_status pa_bm_append(pa_block_manager* m, int32_t seq, int32_t token, int32_t* slot,
                       int32_t* copy_src, int32_t* copy_dst) {
  if (!m || !slot || !copy_src || !copy_dst) return PA_ERR_NULL;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_SHAPE;
  Seq& s = it->second;
  const int bs = m->bs;
  const int64_t p = static_cast<int64_t>(s.tokens.size());
  if (p >= INT32_MAX) return PA_ERR_SHAPE;
  *copy_src = *copy_dst = -1;
  if (p % bs == 0) {
    if (m->available() < 1) return PA_ERR_OUT_OF_BLOCKS;
    s.table.push_back(m->take());
  } else {
    const int32_t last = s.table[p / bs];
    if (m->refs[last] > 1) {
      if (m->available() < 1) return PA_ERR_OUT_OF_BLOCKS;
      const int32_t b = m->take();
      --m->refs[last];
      s.table[p / bs] = b;
      *copy_src = last;
      *copy_dst = b;
    }
  }
  s.tokens.push_back(token);
  *slot = s.table[p / bs] * bs + static_cast<int32_t>(p % bs);
  if ((p + 1) % bs == 0 && m->caching) {
    const int64_t j = p / bs;
    const uint64_t par = j > 0 ? s.keys[j - 1] : kFnvOffset;
    const int32_t* toks = s.tokens.data() + j * bs;
    const uint64_t k = fnv1a(par, toks, bs);
    s.keys.push_back(k);
    m->register_key(s.table[j], k, par, toks);
  }
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* m, int32_t seq, int32_t* new_seq) {
  if (!m || !new_seq) return PA_ERR_NULL;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_SHAPE;
  Seq copy = it->second;
  for (int32_t b : copy.table) ++m->refs[b];
  const int32_t id = m->next_id++;
  m->seqs.emplace(id, std::move(copy));
  *new_seq = id;
  return PA_OK;
}

pa_status pa_bm_free(pa_block_manager* m, int32_t seq) {
  if (!m) return PA_ERR_NULL;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_SHAPE;
  const std::vector<int32_t>& t = it->second.table;
  for (auto r = t.rbegin(); r != t.rend(); ++r) m->release(*r);
  m->seqs.erase(it);
  return PA_OK;
}

int32_t pa_bm_table(const pa_block_manager* m, int32_t seq, int32_t* out, int32_t capacity) {
  if (!m) return -1;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return -1;
  const std::vector<int32_t>& t = it->second.table;
  const int32_t n = static_cast<int32_t>(t.size());
  for (int32_t i = 0; out && i < n && i < capacity; ++i) out[i] = t[i];
  return n;
}

int32_t pa_bm_length(const pa_block_manager* m, int32_t seq) {
  if (!m) return -1;
  auto it = m->seqs.find(seq);
  return it == m->seqs.end() ? -1 : static_cast<int32_t>(it->second.tokens.size());
}

int32_t pa_bm_free_blocks(const pa_block_manager* m) { return m ? m->available() : -1; }

int32_t pa_bm_cached_blocks(const pa_block_manager* m) {
  return m ? static_cast<int32_t>(m->owner.size()) : -1;
}

}  // extern "C"
