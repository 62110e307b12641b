/*
 * pagedkv_blocks.h -- host-side block manager of libpagedkv.so (plain C++,
 * host memory only, no GPU calls) and the device copy used for copy-on-write.
 *
 * Page "Serving LLMs with vLLM: Continuous Batching and PagedAttention
 * Explained":
 *   - "Blocks and Block Tables": the KV cache is cut into fixed-size blocks;
 *     each sequence has a table of the physical blocks holding its logical
 *     blocks; a new block is taken from the free list only when the current
 *     one is full;
 *   - "Growing During Decode": each step appends tokens into the last block,
 *     a full block gets a successor from the free list, and a finished
 *     sequence returns all its blocks to the free pool at once;
 *   - "Shared Prefixes" / "The Savings in Numbers": sequences with an
 *     identical prefix point their tables at the same physical blocks, each
 *     block carrying a reference count;
 *   - "Copy-on-Write": writing into a block whose reference count is above one
 *     first copies it to a fresh block, and only the writer's table changes
 *     (this is also how several samples of one prompt diverge).  With the
 *     prefix cache on, a block that is the value of a key is copied before
 *     any write into it even when its writer is its only reader: a key names
 *     the block's exact tokens, so a cached block never changes;
 *   - "What the Scheduler Does": a sequence is admitted only if enough blocks
 *     are free; a sequence can be preempted by releasing its blocks.
 *
 * Page "Why a Second Kind of Engine", section "Prefix caching" (and the quiz
 * question there on a request id placed before a shared tool schema): every
 * full block is keyed by a hash of its own tokens chained with the key of the
 * block before it; keys map to cached blocks, which are evicted least recently
 * used first when space runs out, and a new request whose leading blocks match
 * cached keys takes those blocks instead of prefilling them.
 *
 * A sequence is named by a caller-chosen int64 id.  All pointers below are HOST
 * memory unless marked device.  Functions return a pkv_status (pagedkv.h);
 * PKV_ERR_SHAPE also reports an unknown or duplicate sequence id and
 * PKV_ERR_WORKSPACE an exhausted free list (nothing is changed in that case).
 * A manager is not thread-safe: one thread drives it.
 */
#ifndef PAGEDKV_BLOCKS_H
#define PAGEDKV_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

/* pkv_bm_create -- a manager of blocks 0 .. num_blocks-1 of block_size tokens, all
 * free; NULL if the sizes are not positive or memory is short.  Blocks are handed
 * out in increasing id order from a fresh manager, freed blocks are reused first
 * (last freed, first reused). */
pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size);
void pkv_bm_destroy(pkv_block_manager* bm);

/* blocks available to new content: free ones plus cached ones that no sequence
 * holds (those are evicted on demand); -1 for a NULL manager */
int32_t pkv_bm_free_blocks(const pkv_block_manager* bm);
/* reference count of a block (0 = free, or cached with no reader); -1 if out of range */
int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block);

/* pkv_bm_add -- a new sequence `seq`.  parent < 0: empty.  Otherwise the new
 * sequence starts with the first shared_tokens tokens of `parent` (0 <=
 * shared_tokens <= parent's length) by pointing its table at the parent's first
 * ceil(shared_tokens / block_size) blocks and raising their reference counts;
 * no block is taken from the free list. */
int pkv_bm_add(pkv_block_manager* bm, int64_t seq, int64_t parent, int32_t shared_tokens);

/* pkv_bm_blocks_needed -- free blocks that appending `counts[i]` tokens to each
 * seqs[i] would take (new blocks plus copy-on-write copies), in *needed. */
int pkv_bm_blocks_needed(const pkv_block_manager* bm, const int64_t* seqs, const int32_t* counts,
                         int32_t n, int32_t* needed);

/* pkv_bm_append -- append counts[i] tokens to each seqs[i], in order.  Writes the
 * slot (block * block_size + offset) of every new token to `slots`
 * (sum(counts) entries, sequence by sequence) and every copy-on-write copy as a
 * (source, destination) block pair to `copies` (at most max_copies pairs; their
 * number in *num_copies).  The copies must reach the device pools
 * (paged_kv_copy_blocks) before the new rows are written.  All or nothing: if
 * the free list cannot cover the whole call, PKV_ERR_WORKSPACE and no change. */
int pkv_bm_append(pkv_block_manager* bm, const int64_t* seqs, const int32_t* counts, int32_t n,
                  int32_t* slots, int32_t* copies, int32_t max_copies, int32_t* num_copies);

/* pkv_bm_release -- drop a finished or preempted sequence: every block's
 * reference count falls by one and blocks reaching zero return to the free list. */
int pkv_bm_release(pkv_block_manager* bm, int64_t seq);

/* pkv_bm_length -- tokens held by a sequence, in *len. */
int pkv_bm_length(const pkv_block_manager* bm, int64_t seq, int32_t* len);

/* pkv_bm_tables -- block tables and lengths of n sequences, as paged_attn_step
 * reads them: tables [n][max_blocks] (-1 past each sequence's blocks), lens [n].
 * PKV_ERR_SHAPE if a sequence holds more than max_blocks blocks. */
int pkv_bm_tables(const pkv_block_manager* bm, const int64_t* seqs, int32_t n, int32_t max_blocks,
                  int32_t* tables, int32_t* lens);

/* pkv_bm_shared_prefix -- per sequence, the number of leading table entries whose
 * block is held by more than one sequence: the shared_blocks hint of paged_attn_step. */
int pkv_bm_shared_prefix(const pkv_block_manager* bm, const int64_t* seqs, int32_t n,
                         int32_t* shared);

/* ---- prefix cache ------------------------------------------------------------------
 *
 * Key of full block i of a token sequence t (block_size B):
 *   key_i = FNV1a64( le64(key_{i-1}) || le32(t[iB]) || ... || le32(t[iB+B-1]) ),  key_{-1} = 0,
 * with 64-bit FNV-1a (offset basis 0xcbf29ce484222325, prime 0x100000001b3) over
 * bytes.  A key therefore depends on every token up to the block's end.  Only
 * full blocks whose token ids are known are keyed; a lookup also compares the
 * stored tokens and parent key, so a hash collision can not return a wrong block.
 * A cached block keeps its key until it is evicted: when the free list is empty,
 * the least recently released cached block with no reader is reused.  Blocks of
 * a released sequence join that list tail first, so a prefix's tail goes before
 * its head.  The K/V a caller writes must be a function of the token prefix alone
 * (as a model's is) for a cached block to stand in for a prefill. */

/* pkv_bm_enable_prefix_cache -- turn the cache on (before any sequence is added;
 * PKV_ERR_SHAPE otherwise or if already on).  Costs 4*block_size + 34 bytes of host
 * memory per block. */
int pkv_bm_enable_prefix_cache(pkv_block_manager* bm);

/* pkv_bm_add_prompt -- a new sequence whose first num_tokens token ids are known
 * (tokens, host int32).  With the cache on, the sequence starts with the longest
 * run of leading full blocks whose keys are cached, one block fewer if that run
 * covers all num_tokens (at least one token is always left to compute); their
 * reference counts rise.  *cached_tokens = tokens already in the cache
 * (a multiple of B); the sequence's length starts there, and the caller appends
 * the remaining num_tokens - *cached_tokens.  With the cache off: an empty
 * sequence whose tokens are recorded, *cached_tokens = 0. */
int pkv_bm_add_prompt(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                      int32_t* cached_tokens);

/* pkv_bm_extend_tokens -- record the ids of n further tokens of `seq` (e.g. the
 * ones it generates), so that the blocks they fill become cacheable.  Blocks
 * already full when their ids arrive are keyed at once. */
int pkv_bm_extend_tokens(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t n);

/* pkv_bm_cache_stats -- stats[5]: keyed blocks, of those the evictable ones (no
 * reader), full prompt blocks looked up, blocks found, blocks evicted. */
int pkv_bm_cache_stats(const pkv_block_manager* bm, int64_t* stats);

/* pkv_prefix_keys -- keys of the floor(num_tokens / block_size) full blocks of a
 * token sequence (host memory), as the manager computes them. */
int pkv_prefix_keys(const int32_t* tokens, int32_t num_tokens, int32_t block_size, uint64_t* keys);

/* paged_kv_copy_blocks -- device copy for copy-on-write ("Copy-on-Write"): for each
 * pair i, block pairs[2i] of both pools (every kv head, every slot) is copied to
 * block pairs[2i+1], bit for bit, and so are the fp8 scales of the block when
 * k_scale / v_scale are given.  pairs: DEVICE int32 [num_pairs][2]; pairs with an
 * id outside [0, num_blocks) are skipped; destinations must be distinct and no
 * destination may be a source of the same call.  Enqueued on `stream`. */
int paged_kv_copy_blocks(const pkv_pool* pool, void* k_pool, void* v_pool, float* k_scale,
                         float* v_scale, const int32_t* pairs, int32_t num_pairs, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_BLOCKS_H */
