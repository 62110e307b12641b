/*
 * pagedkv.h -- C ABI of libpagedkv.so: one scheduler step of attention over a
 * paged KV cache on an AMD Instinct MI355X (gfx950).
 *
 * What the library computes is defined on the page "Serving LLMs with vLLM:
 * Continuous Batching and PagedAttention Explained":
 *   - section "Blocks and Block Tables": the KV cache is cut into fixed-size
 *     blocks in one shared physical pool; each sequence owns a block table that
 *     lists the physical block holding each of its logical blocks, and the
 *     blocks need not be neighbours;
 *   - section "Growing During Decode": every decode step writes the new token's
 *     key and value into the next slot of the sequence's last block
 *     (paged_kv_append);
 *   - section "Attention Over Scattered Blocks": attention reads each block
 *     through the table from wherever it lies, and the result is ordinary
 *     softmax attention of the query over the whole history (paged_attn_step);
 *   - sections "Prefill Versus Decode" and "Chunked Prefill": one step mixes
 *     decoding sequences (one query row each) with a chunk of a long prompt
 *     (several query rows, causal within the history);
 *   - section "Shared Prefixes": several tables may name the same physical
 *     blocks; nothing here writes to them.
 * The 8-bit KV cache ("Why a Second Kind of Engine", section "The memory that
 * concurrency actually costs") is stored as OCP FP8 E4M3FN bytes with one
 * float32 scale per (block, kv head).
 *
 * Conventions for every entry point
 *   Pointers are DEVICE memory owned by the caller unless marked "host".
 *   The library never allocates, frees or synchronises: it validates the host
 *   arguments, enqueues kernels on `stream` (a hipStream_t; NULL = the null
 *   stream) and returns.  Results are valid once the stream has passed the
 *   work; the caller keeps every buffer alive until then.
 *   Return value: a pkv_status (0 = PKV_OK).  Validation failures return before
 *   anything is enqueued.  A failed launch returns PKV_ERR_HIP.  No exception or
 *   abort crosses the ABI.
 *   Device-resident metadata is the caller's contract and is not read back:
 *   block ids in [0, num_blocks), context_lens[i] >= 1 and
 *   <= max_blocks_per_seq * block_size, 1 <= query_lens[i] <= context_lens[i],
 *   append slots distinct.  Kernels skip any address that would fall outside
 *   the pools (so a violation gives wrong numbers, not a memory fault); the
 *   checks build (below) records violations of the attention step's metadata.
 *   Calls are reentrant; calls that share output buffers on concurrent streams
 *   race.  The only process-wide settings are the plan override
 *   (pkv_set_plan_override) and kernel timing (pkv_timing_*), both meant for
 *   tests and measurement.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
typedef enum pkv_dtype {
  PKV_F16 = 0,       /* IEEE binary16 */
  PKV_BF16 = 1,      /* bfloat16 */
  PKV_FP8_E4M3 = 2   /* OCP E4M3FN byte, value = e4m3(byte) * scale[block][kv_head] */
} pkv_dtype;

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,         /* a required pointer is NULL */
  PKV_ERR_SHAPE = 2,        /* a size is out of range or inconsistent */
  PKV_ERR_DTYPE = 3,        /* dtype code unknown or combination not allowed */
  PKV_ERR_WORKSPACE = 4,    /* workspace missing or smaller than paged_attn_workspace_bytes */
  PKV_ERR_UNSUPPORTED = 5,  /* valid request this build has no kernel for */
  PKV_ERR_HIP = 6,          /* the HIP runtime refused a launch */
  PKV_ERR_SCRATCH = 7       /* paged_attn_step_noalloc: the step needs more than its scratch */
} pkv_status;

/* Shape of one layer's K and V pools (host struct).
 * Layout of each pool: [num_blocks][num_kv_heads][block_size][head_dim], elements of
 * kv_dtype, row-major, so one (block, kv head) is one contiguous run of
 * block_size * head_dim elements.
 * Supported: block_size == 16, head_dim in {64, 128}, num_kv_heads >= 1;
 * num_blocks * block_size and num_blocks * num_kv_heads must each fit an int32
 * (PKV_ERR_SHAPE otherwise).
 * Placement (performance only): K and V are separate pointers and may live
 * anywhere, but when a block's K and V slices sit at the same address modulo
 * 2 MiB -- as two separate large allocations put them -- their reads contend
 * for the same HBM banks; starting V an odd multiple of 4 KiB away (e.g. one
 * allocation, V 4 KiB past the end of K) read the 7B-shape decode step's KV
 * about 3% faster on an MI355X. */
typedef struct pkv_pool {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t kv_dtype;         /* pkv_dtype */
} pkv_pool;

/* paged_kv_append -- write this step's new K/V rows into their slots
 * ("Growing During Decode").
 *   pool           host; shape of the pools.
 *   k_pool, v_pool pools to write into (see pkv_pool for the layout).
 *   k_new, v_new   [num_tokens][num_kv_heads][head_dim] rows, elements of new_dtype.
 *   new_dtype      must equal pool->kv_dtype (rows are copied bit for bit; for fp8
 *                  pools the caller has quantised them with the block's scale).
 *   slot_mapping   [num_tokens] int32; slot = block * block_size + offset; a negative
 *                  slot skips its row; slots >= num_blocks * block_size are skipped.
 *   num_tokens     >= 0 (0 enqueues nothing).
 * Bytes of the pools outside the named slots are left untouched.  Must be
 * enqueued before the paged_attn_step that reads the rows (same stream). */
int paged_kv_append(const pkv_pool* pool, void* k_pool, void* v_pool,
                    const void* k_new, const void* v_new, int32_t new_dtype,
                    const int32_t* slot_mapping, int32_t num_tokens, void* stream);

/* paged_kv_append_quant -- append 16-bit rows into an fp8-e4m3 pool, quantising
 * on the way in (the 8-bit cache of "Why a Second Kind of Engine", section "The
 * memory that concurrency actually costs", filled the way "Growing During
 * Decode" fills a block).
 *   k_scale, v_scale  [num_blocks][num_kv_heads] float32 scales of the pools
 *                     (read, and written for new blocks).
 *   k_new, v_new      [num_tokens][num_kv_heads][head_dim], new_dtype PKV_F16 or PKV_BF16.
 *   new_block_k_scale, new_block_v_scale  [num_kv_heads] float32, or both NULL: every
 *                     block whose slot 0 (offset 0) is written by this call first takes
 *                     these per-head scales; other rows use their block's stored scale.
 *   slot_mapping      as paged_kv_append.
 * Each value is divided by its block's scale in IEEE float32 and rounded to the
 * nearest E4M3FN value (ties to even), saturating at +-448 (NaN stays NaN).
 * pool->kv_dtype must be PKV_FP8_E4M3. */
int paged_kv_append_quant(const pkv_pool* pool, void* k_pool, void* v_pool, float* k_scale,
                          float* v_scale, const void* k_new, const void* v_new, int32_t new_dtype,
                          const float* new_block_k_scale, const float* new_block_v_scale,
                          const int32_t* slot_mapping, int32_t num_tokens, void* stream);

/* paged_attn_workspace_bytes -- device scratch paged_attn_step needs for these
 * host scalars (split-context partial results and query row offsets).  Returns 0
 * if the arguments are invalid. */
size_t paged_attn_workspace_bytes(const pkv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t total_q_tokens, int32_t max_context_len,
                                  int32_t max_query_len);

/* paged_attn_step -- attention of every query row of the step over its
 * sequence's paged history ("Attention Over Scattered Blocks").
 *   pool            host; shape of the pools.
 *   q               [total_q_tokens][num_q_heads][head_dim], q_dtype (PKV_F16 or PKV_BF16);
 *                   the query_lens[i] rows of sequence i follow those of sequence i-1.
 *   num_q_heads     multiple of pool->num_kv_heads; query head h reads kv head
 *                   h / (num_q_heads / num_kv_heads).
 *   k_pool, v_pool  the pools, already holding this step's appended rows.
 *   k_scale, v_scale  [num_blocks][num_kv_heads] float32, required iff kv_dtype is
 *                   PKV_FP8_E4M3 (else ignored, may be NULL).
 *   block_tables    [num_seqs][max_blocks_per_seq] int32 physical block ids; entries past
 *                   ceil(context_lens[i] / block_size) are never read.
 *   context_lens    [num_seqs] int32: tokens sequence i attends over, counting the rows
 *                   appended this step.
 *   query_lens      [num_seqs] int32: query rows of sequence i (1 = decode).  Row r sits at
 *                   position context_lens[i] - query_lens[i] + r and attends to keys
 *                   0 .. that position (causal).
 *   shared_blocks   [num_seqs] int32 or NULL: a cache-policy hint.  The first
 *                   shared_blocks[i] table entries of sequence i may also be read by
 *                   other sequences of this step ("Shared Prefixes"; e.g. the leading
 *                   blocks whose reference count is above one); the decode kernel keeps
 *                   those in the caches and streams every other block past them
 *                   (nontemporal loads).  NULL: no block is read twice.  Results do not
 *                   depend on it; a wrong hint only costs bandwidth.
 *   num_seqs, total_q_tokens, max_context_len, max_query_len  host copies of
 *                   len(context_lens), sum(query_lens), max(context_lens), max(query_lens);
 *                   they size the launch grids and must bound the device values.
 *   scale           softmax scale, finite and >= 0 (typically 1/sqrt(head_dim));
 *                   otherwise PKV_ERR_SHAPE.
 *   out             [total_q_tokens][num_q_heads][head_dim], q_dtype, rounded to nearest even.
 *   workspace       device scratch of at least paged_attn_workspace_bytes(...) bytes
 *                   (may be NULL when that is 0); clobbered.
 * Slots of a block past context_lens[i] are never mixed into the result, whatever
 * they hold (they are masked by selection, not by multiplying with zero).
 * PKV_ERR_UNSUPPORTED when one row's split-context partials over all heads
 * (num_q_heads * partitions * head_dim float32, partitions =
 * ceil(max_context_len / partition), one more where split decode rows run as
 * MFMA tiles, whose partition 0 is half a partition long) would pass 2^31
 * bytes. */
int paged_attn_step(const pkv_pool* pool,
                    const void* q, int32_t q_dtype, int32_t num_q_heads,
                    const void* k_pool, const void* v_pool,
                    const float* k_scale, const float* v_scale,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, const int32_t* query_lens,
                    const int32_t* shared_blocks,
                    int32_t num_seqs, int32_t total_q_tokens,
                    int32_t max_context_len, int32_t max_query_len,
                    float scale, void* out,
                    void* workspace, size_t workspace_bytes, void* stream);

/* paged_append_attn_step -- the step's append and its attention in one call
 * ("Growing During Decode" then "Attention Over Scattered Blocks"): the same
 * results as paged_kv_append(pool, k_pool, v_pool, k_new, v_new,
 * pool->kv_dtype, slot_mapping, total_q_tokens) followed by paged_attn_step
 * with the remaining arguments on the same stream, provided that (as in any
 * step a block manager produces) row r's slot is the one block_tables names
 * for that row's position and no other row's context reaches an appended slot.
 *   k_new, v_new    [total_q_tokens][num_kv_heads][head_dim] rows of pool->kv_dtype,
 *                   one per query row, in query-row order.
 *   slot_mapping    [total_q_tokens] int32, as paged_kv_append.
 *   the rest        as paged_attn_step.
 * Decode-only steps (max_query_len 1) of 16-bit KV whose rows run on the VALU
 * decode kernel (at most two query heads per kv head) take the append into the
 * attention launches: the decode launch attends to each new row from k_new /
 * v_new, after the pool's blocks, and the merge launch that follows it (in a
 * step without one, the decode launch) stores the rows into their slots, which
 * saves the append kernel's launch; the pools come out bit for bit the same and
 * the output the same up to that order's rounding.  Split decode-only steps on
 * the MFMA decode kernel (more query heads per kv head, or fp8 KV) leave key
 * L-1 out of the decode launch; the merge launch adds it from k_new / v_new
 * (fp8 rows dequantised with the scales of the block they go to) and stores the
 * rows.  Steps with prefill chunks (max_query_len > 1) of 16-bit KV store the
 * rows from the launch that lists the chunks, before the attention reads them
 * (output bit for bit the two calls').  Every other step (unsplit MFMA decode
 * steps, fp8 steps with prefill chunks) enqueues the append kernel first.
 * Returns the first failing check of either call before anything is enqueued. */
int paged_append_attn_step(const pkv_pool* pool, void* k_pool, void* v_pool,
                           const void* k_new, const void* v_new, const int32_t* slot_mapping,
                           const void* q, int32_t q_dtype, int32_t num_q_heads,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, const int32_t* query_lens,
                           const int32_t* shared_blocks, int32_t num_seqs,
                           int32_t total_q_tokens, int32_t max_context_len,
                           int32_t max_query_len, float scale, void* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* pkv_set_plan_override -- force parts of the launch plan that the library
 * otherwise derives from the host scalars of a step (a testing and tuning
 * hook: every choice gives the same results up to rounding order).
 *   part_tokens        tokens per split-context partition of decode rows (where
 *                      split decode rows run as MFMA tiles, partition 0 holds
 *                      half that, rounded down to a multiple of 16);
 *   chunk_part_tokens  tokens per partition of prefill-chunk rows;
 *                      each 0 (library's choice) or a multiple of 16 in [16, 4096];
 *   small_q            sequences with query_len <= small_q run as decode items
 *                      (applied only where small_q * (num_q_heads / num_kv_heads)
 *                      <= 16); 0 = library's choice, at most 16;
 *   decode_on_mfma     1: decode rows on the MFMA tile kernel, 0: decode-only
 *                      steps run them on the VALU kernel (steps with prefill
 *                      chunks keep fp8 and grouped-query decode rows on the
 *                      MFMA tiles), -1 = library's choice.
 * o == NULL restores every default.  Returns PKV_ERR_SHAPE (and changes
 * nothing) for an out-of-range field.  The setting is process-wide and applies
 * to every later paged_attn_workspace_bytes and paged_attn_step call; set it
 * while no other thread is calling the library, and size the workspace after
 * setting it (a step whose plan needs more workspace than it was given
 * returns PKV_ERR_WORKSPACE). */
typedef struct pkv_plan_override {
  int32_t part_tokens;
  int32_t chunk_part_tokens;
  int32_t small_q;
  int32_t decode_on_mfma;
} pkv_plan_override;
int pkv_set_plan_override(const pkv_plan_override* o);

/* ---- checks build ----
 * libpagedkv_checks.so is this library built with PKV_CHECKS: the same entry
 * points and kernels, plus a validation kernel that paged_attn_step launches
 * first.  It reads the step's device-resident metadata -- context_lens,
 * query_lens and every block_tables entry a context reaches -- against the
 * contract above ("Blocks and Block Tables": a table entry names a block of
 * the pool; "Attention Over Scattered Blocks": a context fits its table and
 * query rows sit at its end) and writes a record into the first
 * PKV_CHECK_RECORD_BYTES bytes of the workspace (paged_attn_workspace_bytes
 * counts them, so a workspace is always needed):
 *   int32 [0] code (pkv_violation), [1] sequence, [2] table column (-1 for a
 *   length), [3] offending value, [4] number of violations found.
 * When several are found, which one is recorded is unspecified.  The step
 * then runs as in the ordinary build (the attention kernels skip what the
 * contract rules out, so other sequences' rows are unaffected).  The record is
 * valid once the stream has passed the step.  pkv_checks_enabled() returns 1
 * in the checks build and 0 in the ordinary one. */
#define PKV_CHECK_RECORD_BYTES 20
typedef enum pkv_violation {
  PKV_VIOLATION_NONE = 0,
  PKV_VIOLATION_BLOCK_ID = 1,      /* an entry within ceil(L/16) outside [0, num_blocks) */
  PKV_VIOLATION_CONTEXT_LEN = 2,   /* L < 1, L > max_blocks_per_seq * 16 or L > max_context_len */
  PKV_VIOLATION_QUERY_LEN = 3,     /* Q < 1, Q > L or Q > max_query_len */
  PKV_VIOLATION_TOTAL_ROWS = 4     /* sum of query_lens != total_q_tokens (sequence -1) */
} pkv_violation;
int pkv_checks_enabled(void);

/* paged_attn_step_noalloc -- paged_attn_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments, kernels and results, but no
 * workspace argument.  The workspace lives in a device array inside the
 * library, paged_attn_scratch_bytes() (64 MiB) long, of which every device the
 * library runs on holds one copy until the process ends; the call itself
 * allocates nothing.  The array used is that of the device `stream` belongs
 * to (the current device for the null stream).  A step whose paged_attn_workspace_bytes exceeds it
 * returns PKV_ERR_SCRATCH before anything is enqueued.  Every call on a device
 * shares that device's array and nothing in it needs to start at zero, so
 * calls on one device whose executions overlap (different streams, or
 * different host threads) race and give wrong results: serialise them (one
 * stream) or use paged_attn_step with a workspace per stream. */
int paged_attn_step_noalloc(const pkv_pool* pool,
                            const void* q, int32_t q_dtype, int32_t num_q_heads,
                            const void* k_pool, const void* v_pool,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, const int32_t* query_lens,
                            const int32_t* shared_blocks,
                            int32_t num_seqs, int32_t total_q_tokens,
                            int32_t max_context_len, int32_t max_query_len,
                            float scale, void* out, void* stream);

/* paged_attn_scratch_bytes -- size of paged_attn_step_noalloc's device scratch. */
size_t paged_attn_scratch_bytes(void);

/* pkv_status_string -- static text for a status code (never NULL). */
const char* pkv_status_string(int status);

/* pkv_last_hip_error / pkv_last_hip_error_string -- the hipError_t (and its name)
 * behind the most recent PKV_ERR_HIP returned on the calling thread; 0 / "hipSuccess"
 * if there was none.  The string is static. */
int pkv_last_hip_error(void);
const char* pkv_last_hip_error_string(void);

/* ---- kernel timing (measurement support, not part of the computation) ----
 * While enabled, every kernel the library enqueues is bracketed by a pair of
 * hipEvents on its own stream.  pkv_timing_enable(capacity) creates `capacity`
 * event pairs up front (host call, allocates) and clears the totals;
 * pkv_timing_disable() destroys them.  pkv_timing_collect() waits for the
 * recorded events, adds their durations to per-kernel totals and recycles the
 * events; pkv_timing_get() returns the total milliseconds and launch count of
 * one kernel kind.  Launches beyond capacity between two collects are not
 * timed (pkv_timing_collect returns how many were dropped). */
typedef enum pkv_kernel_kind {
  PKV_KERNEL_APPEND = 0,       /* kv_append_kernel */
  PKV_KERNEL_PROLOGUE = 1,     /* step_prologue_kernel: row offsets, prefill tile list */
  PKV_KERNEL_DECODE = 2,       /* decode_valu_kernel: decode rows, 16-bit KV, <= 2 heads per kv head */
  PKV_KERNEL_REDUCE = 3,       /* split_reduce_kernel */
  PKV_KERNEL_STEP_MFMA = 4,    /* step_mfma_kernel: prefill-chunk tiles and decode rows in one launch
                                  (steps where some query_len > 1) */
  PKV_KERNEL_DECODE_MFMA = 5,  /* decode_mfma_kernel: grouped-query or fp8 decode rows */
  PKV_KERNEL_KINDS = 6
} pkv_kernel_kind;

int pkv_timing_enable(int32_t capacity);
int pkv_timing_disable(void);
int pkv_timing_collect(int64_t* dropped /* host, may be NULL */);
int pkv_timing_get(int32_t kind, double* total_ms /* host */, int64_t* launches /* host */);

/* pkv_kernel_name -- static name of a pkv_kernel_kind's kernel (never NULL). */
const char* pkv_kernel_name(int32_t kind);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */
