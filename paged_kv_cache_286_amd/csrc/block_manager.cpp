// Host block manager: free list, per-sequence block tables, reference counts,
// prefix sharing and copy-on-write.  Plain C++ over host memory; the only
// device work it implies (copying a block) is paged_kv_copy_blocks in
// copy_blocks.hip.  The contract of every function is in
// include/pagedkv_blocks.h.
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv_blocks.h"

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t len = 0;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_list;     // stack: back() is handed out next
  std::vector<int32_t> ref;           // reference count per block
  std::unordered_map<int64_t, Seq> seqs;
};

namespace {

using Seq = pkv_block_manager::Seq;

int32_t blocks_for(int64_t tokens, int32_t bs) { return (int32_t)((tokens + bs - 1) / bs); }

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
      if (r > 1) {
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
  return bm == nullptr ? -1 : (int32_t)bm->free_list.size();
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
  if (need > (int64_t)bm->free_list.size()) return PKV_ERR_WORKSPACE;
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
      if (bm->ref[last] > 1) {
        const int32_t fresh = bm->free_list.back();
        bm->free_list.pop_back();
        bm->ref[fresh] = 1;
        bm->ref[last] -= 1;
        copies[2 * nc] = last;
        copies[2 * nc + 1] = fresh;
        ++nc;
        last = fresh;
      }
    }
    for (int32_t t = 0; t < counts[i]; ++t) {
      const int32_t pos = s.len + t;
      const int32_t bi = pos / bs;
      if (bi >= (int32_t)s.blocks.size()) {
        const int32_t fresh = bm->free_list.back();
        bm->free_list.pop_back();
        bm->ref[fresh] = 1;
        s.blocks.push_back(fresh);
      }
      slots[w++] = s.blocks[bi] * bs + pos % bs;
    }
    s.len += counts[i];
  }
  if (num_copies) *num_copies = nc;
  return PKV_OK;
}

int pkv_bm_release(pkv_block_manager* bm, int64_t seq) {
  if (bm == nullptr) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_ERR_SHAPE;
  // blocks return in reverse table order, so the sequence's first block is reused first
  for (auto b = it->second.blocks.rbegin(); b != it->second.blocks.rend(); ++b) {
    if (--bm->ref[*b] == 0) bm->free_list.push_back(*b);
  }
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
