// Host block manager: free list, per-sequence block tables, reference counts,
// prefix sharing, copy-on-write and the prefix cache.  Plain C++ over host
// memory; the only device work it implies (copying a block) is
// paged_kv_copy_blocks in copy_blocks.hip.  The contract of every function is
// in include/pagedkv_blocks.h.
//
// Prefix cache (page "Why a Second Kind of Engine", section "Prefix caching",
// and its quiz question on a prepended request id): a full block is keyed by
// a chain hash of its tokens and the key of the block before it, so a key
// names the whole prefix up to the block's end.  Keys map to blocks; a cached
// block whose reference count falls to zero stays cached, on a
// least-recently-used list, and is evicted only when the free list is empty.
// A lookup also compares the stored tokens and parent key, so a 64-bit
// collision of two different blocks can never hand out the wrong KV.
#include <stdint.h>
#include <string.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv_blocks.h"

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t len = 0;
    std::vector<int32_t> tokens;      // known token ids (prefix cache); may be shorter than len
    int32_t hashed = 0;               // leading full blocks already keyed
    uint64_t last_key = 0;            // key of block hashed-1 (0 before the first block)
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_list;     // stack: back() is handed out next
  std::vector<int32_t> ref;           // reference count per block
  std::unordered_map<int64_t, Seq> seqs;

  // prefix cache, allocated when enabled
  bool caching = false;
  std::unordered_map<uint64_t, int32_t> by_key;   // chain key -> block
  std::vector<uint8_t> in_cache;                  // block is the value of some key
  std::vector<uint64_t> key, parent_key;          // per cached block
  std::vector<int32_t> block_tokens;              // [num_blocks][block_size] per cached block
  std::vector<int32_t> lru_prev, lru_next;        // evictable blocks (cached, ref 0), oldest first
  int32_t lru_head = -1, lru_tail = -1, lru_size = 0;
  int64_t stat_lookups = 0, stat_hits = 0, stat_evictions = 0;
};

namespace {

using Seq = pkv_block_manager::Seq;

int32_t blocks_for(int64_t tokens, int32_t bs) { return (int32_t)((tokens + bs - 1) / bs); }

// 64-bit FNV-1a over the little-endian bytes of the parent key and then of
// each token id: the published Fowler-Noll-Vo construction (offset basis
// 0xcbf29ce484222325, prime 0x100000001b3).
uint64_t chain_key(uint64_t parent, const int32_t* tokens, int32_t n) {
  uint64_t h = 0xcbf29ce484222325ull;
  auto eat = [&h](uint64_t v, int bytes) {
    for (int i = 0; i < bytes; ++i) {
      h ^= (v >> (8 * i)) & 0xffu;
      h *= 0x100000001b3ull;
    }
  };
  eat(parent, 8);
  for (int32_t i = 0; i < n; ++i) eat((uint32_t)tokens[i], 4);
  return h;
}

void lru_unlink(pkv_block_manager* bm, int32_t b) {
  const int32_t p = bm->lru_prev[b], n = bm->lru_next[b];
  (p >= 0 ? bm->lru_next[p] : bm->lru_head) = n;
  (n >= 0 ? bm->lru_prev[n] : bm->lru_tail) = p;
  bm->lru_prev[b] = bm->lru_next[b] = -1;
  --bm->lru_size;
}

void lru_push_back(pkv_block_manager* bm, int32_t b) {
  bm->lru_prev[b] = bm->lru_tail;
  bm->lru_next[b] = -1;
  (bm->lru_tail >= 0 ? bm->lru_next[bm->lru_tail] : bm->lru_head) = b;
  bm->lru_tail = b;
  ++bm->lru_size;
}

// blocks that can be handed out: free, or cached with no reader
int64_t available(const pkv_block_manager* bm) {
  return (int64_t)bm->free_list.size() + bm->lru_size;
}

// a block for new content, reference count 1: the free list first, then the
// least recently used cached block (its key is forgotten)
int32_t take_block(pkv_block_manager* bm) {
  int32_t b;
  if (!bm->free_list.empty()) {
    b = bm->free_list.back();
    bm->free_list.pop_back();
  } else {
    b = bm->lru_head;
    lru_unlink(bm, b);
    bm->by_key.erase(bm->key[b]);
    bm->in_cache[b] = 0;
    ++bm->stat_evictions;
  }
  bm->ref[b] = 1;
  return b;
}

// A block that is the value of a prefix-cache key holds exactly the tokens
// its key names, so no sequence may write into it: a sequence whose partial
// last block is such a block (it shared a parent's full block part-way) copies
// it before appending, even when it is the block's only reader.
bool is_cached(const pkv_block_manager* bm, int32_t b) { return bm->caching && bm->in_cache[b]; }

// a block dropped by one reader
void drop_block(pkv_block_manager* bm, int32_t b) {
  if (--bm->ref[b] > 0) return;
  if (bm->caching && bm->in_cache[b])
    lru_push_back(bm, b);
  else
    bm->free_list.push_back(b);
}

// key every leading full block of s whose tokens are all known
void register_full_blocks(pkv_block_manager* bm, Seq& s) {
  if (!bm->caching) return;
  const int32_t bs = bm->block_size;
  const int32_t full = s.len / bs;
  const int32_t known = (int32_t)(s.tokens.size() / bs);
  for (int32_t i = s.hashed; i < full && i < known; ++i) {
    const int32_t* t = s.tokens.data() + (int64_t)i * bs;
    const uint64_t k = chain_key(s.last_key, t, bs);
    const int32_t b = s.blocks[i];
    if (!bm->in_cache[b] && bm->by_key.find(k) == bm->by_key.end()) {
      bm->by_key.emplace(k, b);
      bm->in_cache[b] = 1;
      bm->key[b] = k;
      bm->parent_key[b] = s.last_key;
      memcpy(bm->block_tokens.data() + (int64_t)b * bs, t, sizeof(int32_t) * bs);
    }
    s.last_key = k;
    s.hashed = i + 1;
  }
}

// Blocks an append of `counts` would take, walking the requests in order so
// that a copy-on-write earlier in the call (which lowers a shared block's
// count) is seen by later requests on the same block.
int simulate(const pkv_block_manager* bm, const int64_t* seqs, const int32_t* counts, int32_t n,
             int64_t* needed, int64_t* cow_copies) {
  struct State { int32_t len; int32_t nblocks; bool last_private; };
  std::unordered_map<int64_t, State> st;
  std::unordered_map<int32_t, int32_t> ref_delta;
  int64_t need = 0, cow = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (counts[i] < 0) return PKV_ERR_SHAPE;
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PKV_ERR_SHAPE;
    auto sit = st.find(seqs[i]);
    if (sit == st.end())
      sit = st.emplace(seqs[i], State{it->second.len, (int32_t)it->second.blocks.size(), false}).first;
    State& s = sit->second;
    if (counts[i] == 0) continue;
    if (s.len % bm->block_size != 0 && !s.last_private) {
      const int32_t last = it->second.blocks[s.len / bm->block_size];
      const int32_t r = bm->ref[last] + ref_delta[last];
      if (r > 1 || is_cached(bm, last)) {
        ++need;
        ++cow;
        ref_delta[last] -= 1;
      }
      s.last_private = true;
    }
    const int32_t total = blocks_for((int64_t)s.len + counts[i], bm->block_size);
    if (total > s.nblocks) {
      need += total - s.nblocks;
      s.nblocks = total;
      s.last_private = true;
    }
    s.len += counts[i];
  }
  *needed = need;
  *cow_copies = cow;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks < 1 || block_size < 1 || (int64_t)num_blocks * block_size > INT32_MAX) return nullptr;
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager();
  if (bm == nullptr) return nullptr;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->ref.assign(num_blocks, 0);
    bm->free_list.reserve(num_blocks);
    for (int32_t b = num_blocks - 1; b >= 0; --b) bm->free_list.push_back(b);
  } catch (...) {
    delete bm;
    return nullptr;
  }
  return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int32_t pkv_bm_free_blocks(const pkv_block_manager* bm) {
  return bm == nullptr ? -1 : (int32_t)available(bm);
}

int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block) {
  if (bm == nullptr || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

int pkv_bm_add(pkv_block_manager* bm, int64_t seq, int64_t parent, int32_t shared_tokens) {
  if (bm == nullptr) return PKV_ERR_NULL;
  if (bm->seqs.count(seq)) return PKV_ERR_SHAPE;
  Seq s;
  if (parent >= 0) {
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end() || shared_tokens < 0 || shared_tokens > it->second.len)
      return PKV_ERR_SHAPE;
    const int32_t nb = blocks_for(shared_tokens, bm->block_size);
    s.blocks.assign(it->second.blocks.begin(), it->second.blocks.begin() + nb);
    s.len = shared_tokens;
  } else if (shared_tokens != 0) {
    return PKV_ERR_SHAPE;
  }
  try {
    bm->seqs.emplace(seq, std::move(s));
  } catch (...) {
    return PKV_ERR_WORKSPACE;
  }
  for (int32_t b : bm->seqs[seq].blocks) bm->ref[b] += 1;
  return PKV_OK;
}

int pkv_bm_enable_prefix_cache(pkv_block_manager* bm) {
  if (bm == nullptr) return PKV_ERR_NULL;
  if (bm->caching || !bm->seqs.empty()) return PKV_ERR_SHAPE;
  try {
    const size_t nb = (size_t)bm->num_blocks;
    bm->in_cache.assign(nb, 0);
    bm->key.assign(nb, 0);
    bm->parent_key.assign(nb, 0);
    bm->block_tokens.assign(nb * (size_t)bm->block_size, 0);
    bm->lru_prev.assign(nb, -1);
    bm->lru_next.assign(nb, -1);
  } catch (...) {
    return PKV_ERR_WORKSPACE;
  }
  bm->caching = true;
  return PKV_OK;
}

int pkv_bm_add_prompt(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                      int32_t* cached_tokens) {
  if (bm == nullptr || cached_tokens == nullptr || (num_tokens > 0 && tokens == nullptr))
    return PKV_ERR_NULL;
  if (num_tokens < 0 || bm->seqs.count(seq)) return PKV_ERR_SHAPE;
  const int32_t bs = bm->block_size;
  std::vector<int32_t> hit;
  uint64_t parent = 0;
  if (bm->caching) {
    const int32_t full = num_tokens / bs;
    for (int32_t i = 0; i < full; ++i) {
      const int32_t* t = tokens + (int64_t)i * bs;
      const uint64_t k = chain_key(parent, t, bs);
      auto it = bm->by_key.find(k);
      if (it == bm->by_key.end()) break;
      const int32_t b = it->second;
      if (bm->parent_key[b] != parent ||
          memcmp(bm->block_tokens.data() + (int64_t)b * bs, t, sizeof(int32_t) * bs) != 0)
        break;
      hit.push_back(b);
      parent = k;
    }
    // at least one prompt token is left to compute, so that the step that
    // finishes the prompt has a query row
    if (!hit.empty() && (int64_t)hit.size() * bs >= num_tokens) {
      hit.pop_back();
      parent = hit.empty() ? 0 : bm->key[hit.back()];
    }
    bm->stat_lookups += full;
    bm->stat_hits += (int64_t)hit.size();
  }
  try {
    Seq s;
    s.tokens.assign(tokens, tokens + num_tokens);
    s.blocks = hit;
    bm->seqs.emplace(seq, std::move(s));
  } catch (...) {
    return PKV_ERR_WORKSPACE;
  }
  for (int32_t b : hit) {
    if (bm->ref[b] == 0) lru_unlink(bm, b);
    bm->ref[b] += 1;
  }
  Seq& s = bm->seqs[seq];
  s.len = (int32_t)hit.size() * bs;
  s.hashed = (int32_t)hit.size();
  s.last_key = parent;
  *cached_tokens = s.len;
  return PKV_OK;
}

int pkv_bm_extend_tokens(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t n) {
  if (bm == nullptr || (n > 0 && tokens == nullptr)) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (n < 0 || it == bm->seqs.end()) return PKV_ERR_SHAPE;
  try {
    it->second.tokens.insert(it->second.tokens.end(), tokens, tokens + n);
  } catch (...) {
    return PKV_ERR_WORKSPACE;
  }
  register_full_blocks(bm, it->second);
  return PKV_OK;
}

int pkv_bm_cache_stats(const pkv_block_manager* bm, int64_t* stats) {
  if (bm == nullptr || stats == nullptr) return PKV_ERR_NULL;
  stats[0] = (int64_t)bm->by_key.size();
  stats[1] = bm->lru_size;
  stats[2] = bm->stat_lookups;
  stats[3] = bm->stat_hits;
  stats[4] = bm->stat_evictions;
  return PKV_OK;
}

int pkv_prefix_keys(const int32_t* tokens, int32_t num_tokens, int32_t block_size, uint64_t* keys) {
  if (num_tokens < 0 || block_size < 1) return PKV_ERR_SHAPE;
  const int32_t full = num_tokens / block_size;
  if (full > 0 && (tokens == nullptr || keys == nullptr)) return PKV_ERR_NULL;
  uint64_t parent = 0;
  for (int32_t i = 0; i < full; ++i) {
    parent = chain_key(parent, tokens + (int64_t)i * block_size, block_size);
    keys[i] = parent;
  }
  return PKV_OK;
}

int pkv_bm_blocks_needed(const pkv_block_manager* bm, const int64_t* seqs, const int32_t* counts,
                         int32_t n, int32_t* needed) {
  if (bm == nullptr || needed == nullptr || (n > 0 && (seqs == nullptr || counts == nullptr)))
    return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  int64_t need = 0, cow = 0;
  const int st = simulate(bm, seqs, counts, n, &need, &cow);
  if (st != PKV_OK) return st;
  *needed = (int32_t)need;
  return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* bm, const int64_t* seqs, const int32_t* counts, int32_t n,
                  int32_t* slots, int32_t* copies, int32_t max_copies, int32_t* num_copies) {
  if (bm == nullptr || (n > 0 && (seqs == nullptr || counts == nullptr))) return PKV_ERR_NULL;
  if (n < 0 || max_copies < 0) return PKV_ERR_SHAPE;
  int64_t need = 0, cow = 0;
  const int st = simulate(bm, seqs, counts, n, &need, &cow);
  if (st != PKV_OK) return st;
  if (need > available(bm)) return PKV_ERR_WORKSPACE;
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) total += counts[i];
  if (total > 0 && slots == nullptr) return PKV_ERR_NULL;
  if (cow > 0 && (copies == nullptr || num_copies == nullptr)) return PKV_ERR_NULL;
  if (cow > max_copies) return PKV_ERR_SHAPE;
  // every check passed: this part cannot fail
  const int32_t bs = bm->block_size;
  int32_t nc = 0;
  int64_t w = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = bm->seqs[seqs[i]];
    if (counts[i] == 0) continue;
    if (s.len % bs != 0) {
      int32_t& last = s.blocks[s.len / bs];
      if (bm->ref[last] > 1 || is_cached(bm, last)) {
        const int32_t fresh = take_block(bm);
        drop_block(bm, last);
        copies[2 * nc] = last;
        copies[2 * nc + 1] = fresh;
        ++nc;
        last = fresh;
      }
    }
    for (int32_t t = 0; t < counts[i]; ++t) {
      const int32_t pos = s.len + t;
      const int32_t bi = pos / bs;
      if (bi >= (int32_t)s.blocks.size()) s.blocks.push_back(take_block(bm));
      slots[w++] = s.blocks[bi] * bs + pos % bs;
    }
    s.len += counts[i];
    register_full_blocks(bm, s);
  }
  if (num_copies) *num_copies = nc;
  return PKV_OK;
}

int pkv_bm_release(pkv_block_manager* bm, int64_t seq) {
  if (bm == nullptr) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_ERR_SHAPE;
  // blocks return in reverse table order, so the sequence's first block is reused first
  // (on the least-recently-used list too, so a cached prefix's tail is evicted
  // before its head)
  for (auto b = it->second.blocks.rbegin(); b != it->second.blocks.rend(); ++b) drop_block(bm, *b);
  bm->seqs.erase(it);
  return PKV_OK;
}

int pkv_bm_length(const pkv_block_manager* bm, int64_t seq, int32_t* len) {
  if (bm == nullptr || len == nullptr) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_ERR_SHAPE;
  *len = it->second.len;
  return PKV_OK;
}

int pkv_bm_shared_prefix(const pkv_block_manager* bm, const int64_t* seqs, int32_t n,
                         int32_t* shared) {
  if (bm == nullptr || (n > 0 && (seqs == nullptr || shared == nullptr))) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i)
    if (!bm->seqs.count(seqs[i])) return PKV_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = bm->seqs.at(seqs[i]);
    int32_t k = 0;
    while (k < (int32_t)s.blocks.size() && bm->ref[s.blocks[k]] > 1) ++k;
    shared[i] = k;
  }
  return PKV_OK;
}

int pkv_bm_tables(const pkv_block_manager* bm, const int64_t* seqs, int32_t n, int32_t max_blocks,
                  int32_t* tables, int32_t* lens) {
  if (bm == nullptr || (n > 0 && (seqs == nullptr || tables == nullptr || lens == nullptr)))
    return PKV_ERR_NULL;
  if (n < 0 || max_blocks < 1) return PKV_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end() || (int32_t)it->second.blocks.size() > max_blocks) return PKV_ERR_SHAPE;
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = bm->seqs.at(seqs[i]);
    int32_t* row = tables + (int64_t)i * max_blocks;
    int32_t j = 0;
    for (; j < (int32_t)s.blocks.size(); ++j) row[j] = s.blocks[j];
    for (; j < max_blocks; ++j) row[j] = -1;
    lens[i] = s.len;
  }
  return PKV_OK;
}

}  // extern "C"
