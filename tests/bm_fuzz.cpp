// Random operations on the host block manager, checked against a plain model
// of what the tables must hold; built with the address and undefined-behaviour
// sanitizers by tests/test_block_manager_fuzz.py (host code only).
//
//   bm_fuzz <seed> <operations> <prefix cache 0|1>
//
// A model pool stands in for the K/V pools: appending token p of a sequence
// writes a hash of its token prefix 0..p into the token's slot (K/V are a
// function of the prefix), after the call's copy-on-write copies.  After every
// operation: every live sequence's table covers its length and every one of its
// slots holds its own prefix hash (whatever it shares, forks or finds in the
// prefix cache), each block's reference count equals the number of live tables
// holding it, the blocks available plus the blocks held make up the pool, the
// shared-prefix hint counts the leading entries held more than once, and a
// token appended this step sits in a block no other sequence holds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <map>
#include <vector>

#include "../include/pagedkv_blocks.h"

namespace {

uint64_t rng_state;
uint32_t next_u32() {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (uint32_t)(rng_state >> 11);
}
int below(int n) { return n > 0 ? (int)(next_u32() % (uint32_t)n) : 0; }

constexpr int kBlocks = 64;
constexpr int kB = 16;
constexpr int kMaxBlocks = kBlocks;
constexpr int kVocab = 3;   // few distinct tokens
constexpr int kTexts = 3;   // prompts' common openings

struct Seq {
  std::vector<int32_t> tokens;   // ids of every token (the cache keys need them)
};

// what the K/V of token p of a sequence stand for: a hash of tokens 0..p
uint64_t prefix_hash(const std::vector<int32_t>& t, size_t p) {
  uint64_t h = 1469598103934665603ull;
  for (size_t i = 0; i <= p; ++i) h = (h ^ (uint64_t)(uint32_t)t[i]) * 1099511628211ull;
  return h;
}

int fail(const char* what, long op) {
  fprintf(stderr, "bm_fuzz: %s (operation %ld)\n", what, op);
  return 1;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  rng_state = 0x9E3779B97F4A7C15ull ^ (uint64_t)atoll(argv[1]);
  const long ops = atol(argv[2]);
  const bool cache = atoi(argv[3]) != 0;
  pkv_block_manager* bm = pkv_bm_create(kBlocks, kB);
  if (!bm) return fail("create", -1);
  if (cache && pkv_bm_enable_prefix_cache(bm) != 0) return fail("enable cache", -1);
  std::vector<std::vector<int32_t>> texts(kTexts);
  for (auto& t : texts)
    for (int i = 0; i < 4 * kB; ++i) t.push_back(below(kVocab));
  std::map<int64_t, Seq> live;
  std::vector<uint64_t> pool((size_t)kBlocks * kB, 0);   // the model of the K/V pools
  auto apply_copies = [&](const int32_t* pairs, int32_t n) {
    for (int32_t c = 0; c < n; ++c)
      for (int o = 0; o < kB; ++o) pool[(size_t)pairs[2 * c + 1] * kB + o] = pool[(size_t)pairs[2 * c] * kB + o];
  };
  int64_t next_id = 1;
  std::vector<int32_t> tables, lens, shared;

  for (long op = 0; op < ops; ++op) {
    const int kind = below(10);
    std::vector<int64_t> appended_seqs;
    std::vector<int32_t> appended_slots;
    if (kind <= 1 || live.empty()) {
      // a new sequence: a prompt (its ids known to the cache), then its tokens appended
      const int64_t id = next_id++;
      Seq s;
      // most prompts start with a prefix of one of a few fixed texts (system
      // prompts), so the cache finds keyed blocks
      const int n = 1 + below(4 * kB);
      const int from = below(10) < 7 ? below(n + 1) : 0;
      const int text = below(kTexts);
      for (int i = 0; i < n; ++i) s.tokens.push_back(i < from ? texts[text][i] : below(kVocab));
      int32_t cached = -1;
      if (pkv_bm_add_prompt(bm, id, s.tokens.data(), n, &cached) != 0) return fail("add_prompt", op);
      if (cached < 0 || cached % kB != 0 || cached >= n) return fail("cached tokens", op);
      int32_t len = -1;
      if (pkv_bm_length(bm, id, &len) != 0 || len != cached) return fail("length after add_prompt", op);
      const int32_t count = n - cached;
      std::vector<int32_t> slots(count);
      int32_t copies[2 * 8], nc = -1;
      const int st = pkv_bm_append(bm, &id, &count, 1, slots.data(), copies, 8, &nc);
      if (st == 4) {                         // pool full: nothing changed; drop the sequence
        if (pkv_bm_release(bm, id) != 0) return fail("release after a full pool", op);
        continue;
      }
      if (st != 0) return fail("append of a prompt", op);
      apply_copies(copies, nc);
      for (int32_t j = 0; j < count; ++j) pool[slots[j]] = prefix_hash(s.tokens, (size_t)(cached + j));
      live[id] = s;
      for (int32_t x : slots) { appended_seqs.push_back(id); appended_slots.push_back(x); }
    } else if (kind == 2) {
      // a fork sharing part of a live sequence
      auto it = live.begin();
      std::advance(it, below((int)live.size()));
      int32_t plen = 0;
      if (pkv_bm_length(bm, it->first, &plen) != 0) return fail("length of a parent", op);
      const int32_t share = below(plen + 1);
      const int64_t id = next_id++;
      if (pkv_bm_add(bm, id, it->first, share) != 0) return fail("add with a parent", op);
      Seq s;
      s.tokens.assign(it->second.tokens.begin(), it->second.tokens.begin() + share);
      // the manager learns the ids of the fork's shared tokens too (its cache keys need them)
      if (cache && share > 0 && pkv_bm_extend_tokens(bm, id, s.tokens.data(), share) != 0)
        return fail("extend_tokens of a fork", op);
      live[id] = s;
    } else if (kind <= 6) {
      // a step: a few sequences append a few tokens each
      std::vector<int64_t> seqs;
      std::vector<int32_t> counts;
      for (auto& kv : live)
        if (below(3) == 0 && (int)seqs.size() < 6) {
          seqs.push_back(kv.first);
          counts.push_back(1 + below(kB + 4));
        }
      if (seqs.empty()) continue;
      int32_t need = -1;
      if (pkv_bm_blocks_needed(bm, seqs.data(), counts.data(), (int32_t)seqs.size(), &need) != 0)
        return fail("blocks_needed", op);
      int32_t total = 0;
      for (int32_t c : counts) total += c;
      std::vector<int32_t> slots(total);
      std::vector<int32_t> copies(2 * 64);
      int32_t nc = -1;
      const int free_before = pkv_bm_free_blocks(bm);
      const int st = pkv_bm_append(bm, seqs.data(), counts.data(), (int32_t)seqs.size(),
                                   slots.data(), copies.data(), 64, &nc);
      if (st == 4) {
        if (need <= free_before) return fail("append refused although the blocks were there", op);
        if (pkv_bm_free_blocks(bm) != free_before) return fail("a refused append changed the pool", op);
        continue;
      }
      if (st != 0) return fail("append", op);
      if (need > free_before) return fail("append took more blocks than were free", op);
      apply_copies(copies.data(), nc);
      int k = 0;
      for (size_t i = 0; i < seqs.size(); ++i) {
        Seq& s = live[seqs[i]];
        std::vector<int32_t> ids(counts[i]);
        for (int32_t j = 0; j < counts[i]; ++j) {
          ids[j] = below(kVocab);
          s.tokens.push_back(ids[j]);
          pool[slots[k]] = prefix_hash(s.tokens, s.tokens.size() - 1);
          appended_seqs.push_back(seqs[i]);
          appended_slots.push_back(slots[k++]);
        }
        if (cache && pkv_bm_extend_tokens(bm, seqs[i], ids.data(), counts[i]) != 0)
          return fail("extend_tokens", op);
      }
    } else {
      // a sequence finishes
      auto it = live.begin();
      std::advance(it, below((int)live.size()));
      if (pkv_bm_release(bm, it->first) != 0) return fail("release", op);
      live.erase(it);
    }

    // ---- invariants ----
    const int n = (int)live.size();
    std::vector<int64_t> ids;
    for (auto& kv : live) ids.push_back(kv.first);
    tables.assign((size_t)n * kMaxBlocks, -2);
    lens.assign(n, -2);
    shared.assign(n, -2);
    if (n > 0) {
      if (pkv_bm_tables(bm, ids.data(), n, kMaxBlocks, tables.data(), lens.data()) != 0)
        return fail("tables", op);
      if (pkv_bm_shared_prefix(bm, ids.data(), n, shared.data()) != 0) return fail("shared prefix", op);
    }
    std::vector<int> holders(kBlocks, 0);
    std::map<int64_t, int> row_of;
    for (int i = 0; i < n; ++i) {
      row_of[ids[i]] = i;
      const int32_t L = lens[i];
      const Seq& s = live[ids[i]];
      if (L != (int32_t)s.tokens.size()) return fail("length differs from the model", op);
      for (int32_t q = 0; q < L; ++q)
        if (pool[(size_t)tables[(size_t)i * kMaxBlocks + q / kB] * kB + q % kB] != prefix_hash(s.tokens, q))
          return fail("a slot holds another prefix's K/V", op);
      const int nb = (L + kB - 1) / kB;
      for (int j = 0; j < kMaxBlocks; ++j) {
        const int32_t b = tables[(size_t)i * kMaxBlocks + j];
        if (j < nb) {
          if (b < 0 || b >= kBlocks) return fail("table entry out of the pool", op);
          ++holders[b];
        } else if (b != -1) {
          return fail("table entry past the sequence's blocks", op);
        }
      }
    }
    int held = 0;
    for (int b = 0; b < kBlocks; ++b) {
      if (pkv_bm_refcount(bm, b) != holders[b]) return fail("reference count differs from the tables", op);
      held += holders[b] > 0;
    }
    if (pkv_bm_free_blocks(bm) + held != kBlocks) return fail("available + held != pool", op);
    for (int i = 0; i < n; ++i) {
      const int nb = (lens[i] + kB - 1) / kB;
      int lead = 0;
      while (lead < nb && holders[tables[(size_t)i * kMaxBlocks + lead]] > 1) ++lead;
      if (shared[i] != lead) return fail("shared-prefix hint", op);
    }
    // every token appended this step sits at its position's slot, in a block
    // no other live sequence holds
    for (size_t a = 0; a < appended_seqs.size(); ++a) {
      const int64_t sid = appended_seqs[a];
      if (!live.count(sid)) continue;
      const int i = row_of[sid];
      const int32_t slot = appended_slots[a];
      const int32_t b = slot / kB;
      if (holders[b] != 1) return fail("an appended token in a shared block", op);
      bool found = false;
      for (int j = 0; j < (lens[i] + kB - 1) / kB; ++j)
        if (tables[(size_t)i * kMaxBlocks + j] == b) found = true;
      if (!found) return fail("an appended slot outside the sequence's table", op);
    }
  }
  for (auto& kv : live)
    if (pkv_bm_release(bm, kv.first) != 0) return fail("final release", ops);
  if (pkv_bm_free_blocks(bm) != kBlocks) return fail("blocks lost", ops);
  int64_t stats[5] = {0, 0, 0, 0, 0};
  if (cache && pkv_bm_cache_stats(bm, stats) != 0) return fail("cache stats", ops);
  pkv_bm_destroy(bm);
  printf("bm_fuzz ok: %ld operations, cache %d, %lld cached blocks found\n", ops, (int)cache,
         (long long)stats[3]);
  return 0;
}
