// C ABI of libpagedkv: argument validation, the launch plan of a step, the
// workspace carve-up and optional per-kernel event timing.  See
// include/pagedkv.h for the contract of every entry point.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/pagedkv.h"
#include "pkv_launch.h"

namespace {

using pkv::StepParams;
using pkv::StepPlan;

constexpr int kNumKinds = PKV_KERNEL_KINDS;

// HIP error behind the most recent PKV_ERR_HIP of this thread
thread_local hipError_t g_last_hip_error = hipSuccess;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return PKV_OK;
  g_last_hip_error = e;
  return PKV_ERR_HIP;
}

int elem_bytes(int dtype) { return dtype == PKV_FP8_E4M3 ? 1 : 2; }
bool known_dtype(int d) { return d == PKV_F16 || d == PKV_BF16 || d == PKV_FP8_E4M3; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_pool(const pkv_pool* pool) {
  if (pool == nullptr) return PKV_ERR_NULL;
  if (!known_dtype(pool->kv_dtype)) return PKV_ERR_DTYPE;
  if (pool->num_blocks < 1 || pool->num_kv_heads < 1 || pool->block_size < 1 || pool->head_dim < 1)
    return PKV_ERR_SHAPE;
  if ((int64_t)pool->num_blocks * pool->block_size > INT32_MAX) return PKV_ERR_SHAPE;
  if ((int64_t)pool->num_blocks * pool->num_kv_heads > INT32_MAX) return PKV_ERR_SHAPE;
  if (pool->block_size != 16) return PKV_ERR_UNSUPPORTED;
  if (pool->head_dim != 64 && pool->head_dim != 128) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------
struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> start, stop;
  std::vector<int> pending_kind;   // kind of each recorded pair, in order
  int64_t dropped = 0;
  double total_ms[kNumKinds] = {};
  int64_t launches[kNumKinds] = {};
};
Timing& timing() {
  static Timing t;
  return t;
}

template <class F>
hipError_t timed_launch(int kind, hipStream_t stream, F&& launch) {
  Timing& t = timing();
  int slot = -1;
  {
    std::lock_guard<std::mutex> g(t.mu);
    if (t.on) {
      if (t.pending_kind.size() < t.start.size()) {
        slot = (int)t.pending_kind.size();
        t.pending_kind.push_back(kind);
      } else {
        ++t.dropped;
      }
    }
  }
  if (slot >= 0 && hipEventRecord(t.start[slot], stream) != hipSuccess) return hipErrorUnknown;
  const hipError_t e = launch();
  if (slot >= 0 && hipEventRecord(t.stop[slot], stream) != hipSuccess) return hipErrorUnknown;
  return e;
}

// ---------------------------------------------------------------------------
// the plan of a step
// ---------------------------------------------------------------------------
// Forced plan choices (pkv_set_plan_override); 0 / -1 = the library's own.
struct PlanOverride {
  std::atomic<int32_t> part_tokens{0};
  std::atomic<int32_t> chunk_part_tokens{0};
  std::atomic<int32_t> small_q{0};
  std::atomic<int32_t> decode_on_mfma{-1};
};
PlanOverride& plan_override() {
  static PlanOverride o;
  return o;
}

// Tokens per split-context partition: about 512 KiB (fp8: 1 MiB) of K+V per
// workgroup, halved while a step of few, long rows would leave the chip
// under-filled -- but not below 64 KiB per workgroup: a partition that short
// saves less time than the merge launch it brings costs (a tiny step of 4
// rows of at most 80 tokens runs unsplit, in two launches instead of three).
int32_t part_tokens_for(const pkv_pool* pool, int32_t rows, int32_t wg_per_row, int32_t max_ctx) {
  const int forced = plan_override().part_tokens.load(std::memory_order_relaxed);
  if (forced != 0) return forced;
  const int32_t bytes_per_token = 2 * pool->head_dim * elem_bytes(pool->kv_dtype);
  // fp8 workgroups run the longer MFMA ring; they amortise their start-up over more bytes
  int32_t pt = (pool->kv_dtype == PKV_FP8_E4M3 ? 1024 : 512) * 1024 / bytes_per_token;
  pt = std::min(4096, std::max(16, pt));
  while (pt > 64 && (int64_t)(pt / 2) * bytes_per_token >= 64 * 1024) {
    const int64_t wgs = (int64_t)rows * wg_per_row * ((max_ctx + pt - 1) / pt);
    if (wgs >= 4 * 256) break;
    pt /= 2;
  }
  return pt;
}

// The checks build (compiled with PKV_CHECKS) keeps its violation record in the
// first kCheckBytes of the workspace.
#ifdef PKV_CHECKS
constexpr size_t kCheckBytes = 256;
#else
constexpr size_t kCheckBytes = 0;
#endif

struct Layout {
  size_t q_start_off = 0, row_seq_off = 0, chunk_count_off = 0, chunk_entries_off = 0;
  size_t ml_off = 0, o_off = 0, total = 0;
  int32_t part_tokens = 0, part_head = 0, chunk_part_tokens = 0, max_parts = 0, chunk_max_parts = 0;
  int32_t chunk_capacity = 0, chunk_cols = 64, heads_per_wg = 1, small_q = 1;
  bool decode_on_mfma = false;
};

// Sequences whose query_len * G fits one 16-column tile (a decode, or the few
// rows a speculative-decoding step verifies) run as decode items, their
// blocks shared by the workgroup's four waves; longer prefill chunks become
// chunk entries of chunk_entry_cols columns.
int32_t small_q_for(int32_t group) {
  const int forced = plan_override().small_q.load(std::memory_order_relaxed);
  if (forced >= 1 && forced * group <= 16) return forced;
  return group <= 16 ? std::max(1, 16 / group) : 1;
}

int32_t heads_per_wg_for(int32_t group) {
  for (int g : {8, 4, 2, 1})
    if (group % g == 0) return g;
  return 1;
}

// Decode rows of 16-bit KV with at most two query heads per kv head run on the
// VALU kernel (one token row per 16-lane group, nothing padded); grouped-query
// and fp8 decode rows run on the MFMA tile kernel, where the group's heads fill
// the columns of a 16x16 tile and K/V are read once for all of them.
bool decode_on_mfma_for(const pkv_pool* pool, int32_t group) {
  const int forced = plan_override().decode_on_mfma.load(std::memory_order_relaxed);
  if (forced == 0 || forced == 1) return forced == 1;
  return pool->kv_dtype == PKV_FP8_E4M3 || group > 2;
}

int32_t round16(int64_t x) { return (int32_t)((x + 15) / 16 * 16); }

// Tokens per partition of a prefill-chunk row.  In a step with many
// sequences the decode items fill the launch: no split when the chunk's
// entries already give >= 128 work items, otherwise enough partitions to reach
// ~256.  A step of at most kFewSeqs sequences has too few decode rows to fill
// 256 CUs, so its chunks are split to ~512 items (a lone 512-row chunk over
// 2,560 keys at the 7B shape: 179 us unsplit, 95 us in four partitions).
// At most 4096 (256 blocks per wave).
constexpr int32_t kFewSeqs = 8;
int32_t chunk_part_tokens_for(int32_t group, int32_t num_kv_heads, int32_t max_ctx, int32_t max_q,
                              int32_t cols, int32_t num_seqs) {
  const int forced = plan_override().chunk_part_tokens.load(std::memory_order_relaxed);
  if (forced != 0) return forced;
  const int64_t tiles = ((int64_t)max_q * group + cols - 1) / cols;
  const int64_t items = tiles * num_kv_heads;
  const int64_t want = num_seqs <= kFewSeqs ? 512 : 256;
  int64_t parts = (num_seqs > kFewSeqs && items >= 128) ? 1 : (want + items - 1) / items;
  int32_t pt = round16((max_ctx + parts - 1) / parts);
  return std::min(4096, std::max(64, pt));
}

Layout layout_for(const pkv_pool* pool, int32_t num_seqs, int32_t num_q_heads, int32_t total_q,
                  int32_t max_ctx, int32_t max_q) {
  Layout lay;
  const int32_t group = num_q_heads / pool->num_kv_heads;
  // Steps with prefill chunks run every row in the step kernel; there too the
  // single-row sequences of VALU-decode shapes run as VALU decode workgroups,
  // and every sequence with more rows becomes chunk entries (small_q = 1).
  lay.heads_per_wg = heads_per_wg_for(group);
  lay.decode_on_mfma = decode_on_mfma_for(pool, group) ||
                       (max_q > 1 && (pool->kv_dtype == PKV_FP8_E4M3 || lay.heads_per_wg > 2));
  const int32_t wg_per_row =
      lay.decode_on_mfma ? pool->num_kv_heads * ((group + 15) / 16) : num_q_heads / lay.heads_per_wg;
  // (the tiles per kv head of small-query sequences only add columns, not blocks)
  lay.part_tokens = part_tokens_for(pool, num_seqs, wg_per_row, max_ctx);
  // split steps whose decode rows run as MFMA tiles: a row's partition 0 is
  // half a partition short, so the last items a decode launch deals
  // (partition 0 of every row) are short ones and the launch's tail is short.
  // The MFMA items are long (fp8: 4,096 tokens) on half the VALU kernel's
  // slots; the VALU decode's items are short already, and there the extra
  // partition of each row cost more than the shorter tail saved.  Unsplit
  // steps stay unsplit.
  lay.part_head = lay.decode_on_mfma && max_ctx > lay.part_tokens ? (lay.part_tokens / 2) & ~15 : 0;
  lay.max_parts = (max_ctx + lay.part_head + lay.part_tokens - 1) / lay.part_tokens;
  size_t off = kCheckBytes;
  if (max_q > 1) {
    lay.small_q = lay.decode_on_mfma ? small_q_for(group) : 1;
    lay.chunk_cols = pkv::chunk_entry_cols(pool->kv_dtype);
    lay.chunk_part_tokens =
        chunk_part_tokens_for(group, pool->num_kv_heads, max_ctx, max_q, lay.chunk_cols, num_seqs);
    lay.chunk_max_parts = (max_ctx + lay.chunk_part_tokens - 1) / lay.chunk_part_tokens;
    lay.max_parts = std::max(lay.max_parts, lay.chunk_max_parts);
    // sum over sequences with q > 1 of ceil(q * group / cols) <= total_q * group / cols + num_seqs
    lay.chunk_capacity = (int32_t)(((int64_t)total_q * group + lay.chunk_cols - 1) / lay.chunk_cols + num_seqs);
    lay.q_start_off = off;
    off = round_up(off + sizeof(int32_t) * ((size_t)num_seqs + 1), 256);
    lay.row_seq_off = off;
    off = round_up(off + sizeof(int32_t) * (size_t)total_q, 256);
    lay.chunk_count_off = off;
    off = round_up(off + sizeof(int32_t), 256);
    lay.chunk_entries_off = off;
    off = round_up(off + 2 * sizeof(int32_t) * (size_t)lay.chunk_capacity, 256);
  }
  if (lay.max_parts > 1) {
    const size_t entries = (size_t)total_q * num_q_heads * lay.max_parts;
    lay.ml_off = off;
    off = round_up(off + entries * 2 * sizeof(float), 256);
    lay.o_off = off;
    off = round_up(off + entries * pool->head_dim * sizeof(float), 256);
  }
  lay.total = off;
  return lay;
}

int check_step_scalars(const pkv_pool* pool, int32_t q_dtype, int32_t num_q_heads,
                       int32_t max_blocks, int32_t num_seqs, int32_t total_q, int32_t max_ctx,
                       int32_t max_q) {
  const int st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (q_dtype != PKV_F16 && q_dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (pool->kv_dtype != q_dtype && pool->kv_dtype != PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  if (num_q_heads < 1 || num_q_heads % pool->num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (num_seqs < 0 || total_q < num_seqs || max_blocks < 1) return PKV_ERR_SHAPE;
  if (num_seqs > 0 && (max_ctx < 1 || max_q < 1 || max_q > max_ctx || max_q > total_q))
    return PKV_ERR_SHAPE;
  if ((int64_t)max_ctx > (int64_t)max_blocks * pool->block_size) return PKV_ERR_SHAPE;
  if (num_seqs > 0 && max_q == 1 && total_q != num_seqs) return PKV_ERR_SHAPE;
  if (num_seqs > 0 && max_q > 1 && (int64_t)total_q < (int64_t)num_seqs + max_q - 1) return PKV_ERR_SHAPE;
  // one-dimensional grids of (head group, row) and (head group, sequence) workgroups
  if ((int64_t)total_q * num_q_heads > INT32_MAX) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

// ---------------------------------------------------------------------------
// the no-allocation entry point's workspace
// ---------------------------------------------------------------------------
// paged_attn_step_noalloc keeps its workspace in this array: each device the
// library runs on holds its own copy from the moment the library's code is
// loaded on it until the process ends.  In host code `scratch` only names the
// symbol; its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// ever handed to kernels.  64 MiB covers every decode and mixed step of the
// 7B shape here (a 640-row mixed step needs 41 MiB).
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchAddresses {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};
};
ScratchAddresses& scratch_addresses() {
  static ScratchAddresses a;
  return a;
}

// this device's scratch address, looked up on the first call on the device
// The scratch array of the device `stream` runs on (the current device for
// the null stream).  The first call on a device makes that device current for
// the symbol lookup, then restores the caller's device.
int device_scratch(void* stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_status(e);
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &d);
    if (e != hipSuccess) return hip_status(e);
    dev = d;
  }
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  ScratchAddresses& a = scratch_addresses();
  std::lock_guard<std::mutex> g(a.mu);
  if (a.ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr) return hip_status(hipErrorInvalidSymbol);
    a.ptr[dev] = p;
  }
  *out = a.ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "a size is out of range or inconsistent";
    case PKV_ERR_DTYPE: return "unknown dtype or dtype combination not allowed";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_UNSUPPORTED: return "no kernel for this shape in this build";
    case PKV_ERR_HIP: return "the HIP runtime refused a launch";
    case PKV_ERR_SCRATCH:
      return "the step needs more workspace than paged_attn_step_noalloc's device scratch holds";
    default: return "unknown status";
  }
}

const char* pkv_kernel_name(int32_t kind) {
  switch (kind) {
    case PKV_KERNEL_APPEND: return "kv_append_kernel";
    case PKV_KERNEL_PROLOGUE: return "step_prologue_kernel";
    case PKV_KERNEL_DECODE: return "decode_valu_kernel";
    case PKV_KERNEL_DECODE_MFMA: return "decode_mfma_kernel";
    case PKV_KERNEL_REDUCE: return "split_reduce_kernel";
    case PKV_KERNEL_STEP_MFMA: return "step_mfma_kernel";
    default: return "unknown";
  }
}

}  // extern "C"

namespace {

// Host checks of an append of num_tokens rows of the pool's own element type.
int check_append(const void* k_pool, const void* v_pool, const void* k_new, const void* v_new,
                 const int32_t* slot_mapping, int32_t num_tokens) {
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return PKV_ERR_NULL;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new))
    return PKV_ERR_SHAPE;
  return PKV_OK;
}

hipError_t enqueue_append(const pkv_pool* pool, void* k_pool, void* v_pool, const void* k_new,
                          const void* v_new, const int32_t* slot_mapping, int32_t num_tokens,
                          hipStream_t s) {
  pkv::AppendArgs a;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.elem_bytes = elem_bytes(pool->kv_dtype);
  a.block_size = pool->block_size;
  a.num_blocks = pool->num_blocks;
  return timed_launch(PKV_KERNEL_APPEND, s, [&] { return pkv::launch_append(a, s); });
}

}  // namespace

extern "C" {

int paged_kv_append(const pkv_pool* pool, void* k_pool, void* v_pool, const void* k_new,
                    const void* v_new, int32_t new_dtype, const int32_t* slot_mapping,
                    int32_t num_tokens, void* stream) {
  int st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (!known_dtype(new_dtype)) return PKV_ERR_DTYPE;
  if (new_dtype != pool->kv_dtype) return PKV_ERR_DTYPE;
  st = check_append(k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens);
  if (st != PKV_OK || num_tokens == 0) return st;
  return hip_status(enqueue_append(pool, k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens,
                                   (hipStream_t)stream));
}

int paged_kv_append_quant(const pkv_pool* pool, void* k_pool, void* v_pool, float* k_scale,
                          float* v_scale, const void* k_new, const void* v_new, int32_t new_dtype,
                          const float* new_block_k_scale, const float* new_block_v_scale,
                          const int32_t* slot_mapping, int32_t num_tokens, void* stream) {
  const int st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (pool->kv_dtype != PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  if (new_dtype != PKV_F16 && new_dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_scale || !v_scale || !k_new || !v_new || !slot_mapping)
    return PKV_ERR_NULL;
  if ((new_block_k_scale == nullptr) != (new_block_v_scale == nullptr)) return PKV_ERR_NULL;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new))
    return PKV_ERR_SHAPE;
  pkv::AppendArgs a;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.elem_bytes = 1;
  a.block_size = pool->block_size;
  a.num_blocks = pool->num_blocks;
  const hipStream_t s = (hipStream_t)stream;
  return hip_status(timed_launch(PKV_KERNEL_APPEND, s, [&] {
    return pkv::launch_append_quant(a, new_dtype, k_scale, v_scale, new_block_k_scale,
                                    new_block_v_scale, s);
  }));
}

size_t paged_attn_workspace_bytes(const pkv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t total_q_tokens, int32_t max_context_len,
                                  int32_t max_query_len) {
  if (check_pool(pool) != PKV_OK) return 0;
  if (num_q_heads < 1 || num_q_heads % pool->num_kv_heads != 0) return 0;
  if (num_seqs < 1 || total_q_tokens < num_seqs || max_context_len < 1 || max_query_len < 1) return 0;
  return layout_for(pool, num_seqs, num_q_heads, total_q_tokens, max_context_len, max_query_len).total;
}

// The append that paged_append_attn_step enqueues with the step.
struct FusedAppend {
  void* k_pool;
  void* v_pool;
  const void* k_new;
  const void* v_new;
  const int32_t* slots;
};

// paged_attn_step, paged_attn_step_noalloc (workspace from this device's
// scratch array instead of the caller's) and paged_append_attn_step (fa: the
// step's append goes first, or into the decode launch).
static int attn_step(const pkv_pool* pool, const void* q, int32_t q_dtype, int32_t num_q_heads,
                     const void* k_pool, const void* v_pool, const float* k_scale,
                     const float* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* query_lens,
                     const int32_t* shared_blocks, int32_t num_seqs,
                     int32_t total_q_tokens, int32_t max_context_len, int32_t max_query_len,
                     float scale, void* out, void* workspace, size_t workspace_bytes,
                     bool use_scratch, const FusedAppend* fa, void* stream) {
  int st = check_step_scalars(pool, q_dtype, num_q_heads, max_blocks_per_seq, num_seqs,
                              total_q_tokens, max_context_len, max_query_len);
  if (st != PKV_OK) return st;
  if (fa != nullptr) {
    st = check_append(fa->k_pool, fa->v_pool, fa->k_new, fa->v_new, fa->slots, total_q_tokens);
    if (st != PKV_OK) return st;
  }
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !query_lens || !out)
    return PKV_ERR_NULL;
  if (pool->kv_dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) return PKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool)) return PKV_ERR_SHAPE;
  // the tile kernels take a block's largest scaled score as the largest raw
  // score times the scale, which holds for a finite scale >= 0
  if (!std::isfinite(scale) || scale < 0.f) return PKV_ERR_SHAPE;

  const Layout lay = layout_for(pool, num_seqs, num_q_heads, total_q_tokens, max_context_len,
                                max_query_len);
  // a decode workgroup addresses its heads' partial rows with 32-bit byte
  // offsets from its first head's
  if ((int64_t)num_q_heads * lay.max_parts * pool->head_dim * 4 > INT32_MAX)
    return PKV_ERR_UNSUPPORTED;
  if (use_scratch) {
    if (lay.total > kScratchBytes) return PKV_ERR_SCRATCH;
    st = device_scratch(stream, &workspace);
    if (st != PKV_OK) return st;
    workspace_bytes = kScratchBytes;
  }
  if (lay.total > 0 && (workspace == nullptr || workspace_bytes < lay.total)) return PKV_ERR_WORKSPACE;

  StepPlan plan;
  plan.kv_dtype = pool->kv_dtype;
  plan.q_dtype = q_dtype;
  plan.head_dim = pool->head_dim;
  plan.group = num_q_heads / pool->num_kv_heads;
  plan.heads_per_wg = lay.heads_per_wg;
  plan.decode_on_mfma = lay.decode_on_mfma;
  plan.chunk_grid = 0;
  if (!pkv::decode_supported(plan)) return PKV_ERR_UNSUPPORTED;

  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  const bool multi = max_query_len > 1;
  StepParams p;
  p.q = q;
  p.out = out;
  p.k_pool = reinterpret_cast<const uint8_t*>(k_pool);
  p.v_pool = reinterpret_cast<const uint8_t*>(v_pool);
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.tables = block_tables;
  p.ctx_lens = context_lens;
  p.q_lens = query_lens;
  p.shared_blocks = shared_blocks;
  // When every sequence has max_query_len rows (total_q == num_seqs * max_q) and
  // that exceeds small_q, every row is a prompt row; if their partition covers
  // the whole context no row has partitions to merge and the merge launch (one
  // workgroup per row and four heads) is skipped.
  const bool all_prompt_rows = multi && (int64_t)num_seqs * max_query_len == total_q_tokens &&
                               max_query_len > lay.small_q;
  const bool merge = lay.max_parts > 1 && !(all_prompt_rows && lay.chunk_max_parts == 1);
  // Decode steps of 16-bit KV on the VALU decode kernel take their append: the
  // decode launch attends to the new rows from k_new / v_new, and the merge
  // launch after it (else the decode launch itself) stores them into the pool.
  // Stores inside the decode launch cost its read stream about what the append
  // kernel takes, so a step with a merge launch leaves them to that one: the
  // append kernel's launch is saved either way.
  // Steps with prefill chunks (16-bit KV) store the rows from the prologue
  // launch that runs before their step kernel anyway.
  const bool fuse = fa != nullptr && !multi && !plan.decode_on_mfma && plan.heads_per_wg <= 2 &&
                    pool->kv_dtype != PKV_FP8_E4M3;
  const bool fuse_prologue = fa != nullptr && multi && pool->kv_dtype != PKV_FP8_E4M3;
  // Split decode steps on the MFMA kernel (grouped-query and fp8 KV): the
  // decode launch leaves key L-1 out, every row writes partials, and the
  // merge launch adds that key from k_new / v_new and stores the rows.
  const bool fuse_merge = fa != nullptr && !multi && plan.decode_on_mfma && merge;
  const bool any_fuse = fuse || fuse_prologue || fuse_merge;
  p.k_new = any_fuse ? reinterpret_cast<const uint8_t*>(fa->k_new) : nullptr;
  p.v_new = any_fuse ? reinterpret_cast<const uint8_t*>(fa->v_new) : nullptr;
  p.slots = any_fuse ? fa->slots : nullptr;
  p.append_in_merge = (fuse && merge) || fuse_merge;
  p.new_in_merge = fuse_merge;
  p.kv_fp8 = pool->kv_dtype == PKV_FP8_E4M3;
  p.append_rows = fuse_prologue ? total_q_tokens : 0;
  p.append_row_bytes = pool->head_dim * elem_bytes(pool->kv_dtype);
  p.q_start = multi ? reinterpret_cast<const int32_t*>(ws + lay.q_start_off) : nullptr;
  p.row_seq = multi ? reinterpret_cast<const int32_t*>(ws + lay.row_seq_off) : nullptr;
  p.chunk_count = multi ? reinterpret_cast<const int32_t*>(ws + lay.chunk_count_off) : nullptr;
  p.chunk_entries = multi ? reinterpret_cast<const int32_t*>(ws + lay.chunk_entries_off) : nullptr;
  p.part_ml = lay.max_parts > 1 ? reinterpret_cast<float*>(ws + lay.ml_off) : nullptr;
  p.part_o = lay.max_parts > 1 ? reinterpret_cast<float*>(ws + lay.o_off) : nullptr;
  // fp8 KV: partial outputs as bfloat16 (their rounding, 2^-9 of a partition's
  // output, is far inside what the 3-bit mantissas of the keys and values leave)
  p.part_bf16 = pool->kv_dtype == PKV_FP8_E4M3;
  p.num_blocks = pool->num_blocks;
  p.num_kv_heads = pool->num_kv_heads;
  p.num_q_heads = num_q_heads;
  p.max_blocks = max_blocks_per_seq;
  p.num_seqs = num_seqs;
  p.total_q = total_q_tokens;
  p.max_parts = lay.max_parts;
  p.part_tokens = lay.part_tokens;
  p.part_head = lay.part_head;
  p.chunk_part_tokens = multi ? lay.chunk_part_tokens : lay.part_tokens;
  p.chunk_max_parts = lay.chunk_max_parts;
  p.chunk_capacity = lay.chunk_capacity;
  p.chunk_cols = lay.chunk_cols;
  p.small_q = multi ? lay.small_q : 1;
  p.scale_log2 = scale * pkv::kLog2e;
  if (multi) {
    const int64_t items = (int64_t)lay.chunk_capacity * pool->num_kv_heads * lay.chunk_max_parts;
    plan.chunk_grid = (int32_t)std::min<int64_t>(items, 2048);
  }

  // Steps with prefill chunks run the chunk tiles and the decode rows in one
  // MFMA launch so the chunks' matrix work overlaps the decodes' HBM traffic;
  // decode-only steps pick the VALU or MFMA decode kernel.
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (kCheckBytes > 0)
    e = pkv::launch_check(p, reinterpret_cast<int32_t*>(ws), max_context_len, max_query_len, s);
  if (e == hipSuccess && fa != nullptr && !any_fuse)
    e = enqueue_append(pool, fa->k_pool, fa->v_pool, fa->k_new, fa->v_new, fa->slots,
                       total_q_tokens, s);
  if (e != hipSuccess) return hip_status(e);
  if (multi) {
    e = timed_launch(PKV_KERNEL_PROLOGUE, s, [&] { return pkv::launch_prologue(p, s); });
    if (e == hipSuccess)
      e = timed_launch(PKV_KERNEL_STEP_MFMA, s, [&] { return pkv::launch_step_mfma(p, plan, s); });
  } else {
    e = plan.decode_on_mfma
            ? timed_launch(PKV_KERNEL_DECODE_MFMA, s, [&] { return pkv::launch_decode_mfma(p, plan, s); })
            : timed_launch(PKV_KERNEL_DECODE, s, [&] { return pkv::launch_decode(p, plan, s); });
  }
  if (e == hipSuccess && merge)
    e = timed_launch(PKV_KERNEL_REDUCE, s, [&] { return pkv::launch_reduce(p, plan, s); });
  return hip_status(e);
}

int paged_attn_step(const pkv_pool* pool, const void* q, int32_t q_dtype, int32_t num_q_heads,
                    const void* k_pool, const void* v_pool, const float* k_scale,
                    const float* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, const int32_t* query_lens,
                    const int32_t* shared_blocks, int32_t num_seqs,
                    int32_t total_q_tokens, int32_t max_context_len, int32_t max_query_len,
                    float scale, void* out, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return attn_step(pool, q, q_dtype, num_q_heads, k_pool, v_pool, k_scale, v_scale, block_tables,
                   max_blocks_per_seq, context_lens, query_lens, shared_blocks, num_seqs,
                   total_q_tokens, max_context_len, max_query_len, scale, out, workspace,
                   workspace_bytes, false, nullptr, stream);
}

int paged_append_attn_step(const pkv_pool* pool, void* k_pool, void* v_pool, const void* k_new,
                           const void* v_new, const int32_t* slot_mapping, const void* q,
                           int32_t q_dtype, int32_t num_q_heads, const float* k_scale,
                           const float* v_scale, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           const int32_t* query_lens, const int32_t* shared_blocks,
                           int32_t num_seqs, int32_t total_q_tokens, int32_t max_context_len,
                           int32_t max_query_len, float scale, void* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const FusedAppend fa{k_pool, v_pool, k_new, v_new, slot_mapping};
  return attn_step(pool, q, q_dtype, num_q_heads, k_pool, v_pool, k_scale, v_scale, block_tables,
                   max_blocks_per_seq, context_lens, query_lens, shared_blocks, num_seqs,
                   total_q_tokens, max_context_len, max_query_len, scale, out, workspace,
                   workspace_bytes, false, &fa, stream);
}

int paged_attn_step_noalloc(const pkv_pool* pool, const void* q, int32_t q_dtype,
                            int32_t num_q_heads, const void* k_pool, const void* v_pool,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, const int32_t* query_lens,
                            const int32_t* shared_blocks, int32_t num_seqs,
                            int32_t total_q_tokens, int32_t max_context_len,
                            int32_t max_query_len, float scale, void* out, void* stream) {
  return attn_step(pool, q, q_dtype, num_q_heads, k_pool, v_pool, k_scale, v_scale, block_tables,
                   max_blocks_per_seq, context_lens, query_lens, shared_blocks, num_seqs,
                   total_q_tokens, max_context_len, max_query_len, scale, out, nullptr, 0, true,
                   nullptr, stream);
}

size_t paged_attn_scratch_bytes(void) { return kScratchBytes; }

int pkv_checks_enabled(void) { return kCheckBytes > 0 ? 1 : 0; }

int pkv_set_plan_override(const pkv_plan_override* o) {
  PlanOverride& po = plan_override();
  if (o == nullptr) {
    po.part_tokens = 0;
    po.chunk_part_tokens = 0;
    po.small_q = 0;
    po.decode_on_mfma = -1;
    return PKV_OK;
  }
  auto tokens_ok = [](int32_t t) { return t == 0 || (t >= 16 && t <= 4096 && t % 16 == 0); };
  if (!tokens_ok(o->part_tokens) || !tokens_ok(o->chunk_part_tokens)) return PKV_ERR_SHAPE;
  if (o->small_q < 0 || o->small_q > 16) return PKV_ERR_SHAPE;
  if (o->decode_on_mfma < -1 || o->decode_on_mfma > 1) return PKV_ERR_SHAPE;
  po.part_tokens = o->part_tokens;
  po.chunk_part_tokens = o->chunk_part_tokens;
  po.small_q = o->small_q;
  po.decode_on_mfma = o->decode_on_mfma;
  return PKV_OK;
}

int pkv_timing_enable(int32_t capacity) {
  if (capacity < 1 || capacity > (1 << 20)) return PKV_ERR_SHAPE;
  pkv_timing_disable();
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.start.resize(capacity);
  t.stop.resize(capacity);
  for (int i = 0; i < capacity; ++i) {
    if (hipEventCreate(&t.start[i]) != hipSuccess || hipEventCreate(&t.stop[i]) != hipSuccess) {
      t.start.resize(i);
      t.stop.resize(i);
      return hip_status(hipErrorOutOfMemory);
    }
  }
  t.pending_kind.clear();
  t.dropped = 0;
  for (int k = 0; k < kNumKinds; ++k) { t.total_ms[k] = 0; t.launches[k] = 0; }
  t.on = true;
  return PKV_OK;
}

int pkv_timing_collect(int64_t* dropped) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  for (size_t i = 0; i < t.pending_kind.size(); ++i) {
    hipError_t e = hipEventSynchronize(t.stop[i]);
    if (e != hipSuccess) return hip_status(e);
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, t.start[i], t.stop[i]);
    if (e != hipSuccess) return hip_status(e);
    t.total_ms[t.pending_kind[i]] += ms;
    t.launches[t.pending_kind[i]] += 1;
  }
  t.pending_kind.clear();
  if (dropped) *dropped = t.dropped;
  t.dropped = 0;
  return PKV_OK;
}

int pkv_timing_disable(void) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  for (auto ev : t.start) (void)hipEventDestroy(ev);
  for (auto ev : t.stop) (void)hipEventDestroy(ev);
  t.start.clear();
  t.stop.clear();
  t.pending_kind.clear();
  t.on = false;
  return PKV_OK;
}

int pkv_last_hip_error(void) { return (int)g_last_hip_error; }

const char* pkv_last_hip_error_string(void) { return hipGetErrorName(g_last_hip_error); }

int pkv_timing_get(int32_t kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= kNumKinds) return PKV_ERR_SHAPE;
  if (!total_ms || !launches) return PKV_ERR_NULL;
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  *total_ms = t.total_ms[kind];
  *launches = t.launches[kind];
  return PKV_OK;
}

}  // extern "C"
