// Paged decode attention for gfx950: block-table walk, 16-byte coalesced KV
// loads, fp32 online softmax with DPP reductions, split-context partials.
//
// Page "Serving LLMs with vLLM: Continuous Batching and PagedAttention
// Explained", section "Attention Over Scattered Blocks": the kernel reads the
// block table, fetches each block from its physical place and scores block by
// block; the result is ordinary softmax attention over the whole history.
// Section "Blocks and Block Tables" fixes the addressing: token t of a
// sequence sits in block table[t / 16] at offset t % 16.
//
// Work decomposition (one workgroup = NW wave64s):
//   grid.x  group of `GB` query heads that share one kv head (fastest), then
//           sequence (only sequences with one query row; prefill chunks go to
//           the MFMA chunk kernel) -- one dimension, so the sequence count is
//           not held to grid.y's 65,535,
//   grid.y  split-context partition of part_tokens tokens, in the order
//           set by dispatch_part.
// The hardware deals workgroups to the 8 XCDs round-robin by linear id, so the
// fastest grid dimension must not be one along which the work per workgroup
// changes: heads (equal work) go first and partitions go last.
// Inside a workgroup wave w takes blocks w, w+NW, ... of the partition.  A
// (block, kv head) of K is block_size * head_dim contiguous elements, so one
// wave-wide 16-byte load covers RPL whole token rows with no gaps: lane l
// holds EPL consecutive head dims of token j*RPL + l/LPR.  Each group of LPR
// lanes owning a token row keeps its own running max / sum / accumulator, so
// the per-block softmax needs no cross-row traffic; rows, then waves (through
// LDS), are merged once at the end.  A sequence longer than one partition
// writes (max, sum, unnormalised output) per partition and the reduce kernel
// merges them with the log-sum-exp rule.
#include <type_traits>

#include "decode_valu.h"
#include "pkv_launch.h"

namespace pkv {

// FUSED: the step's append goes into this launch (p.k_new set; 16-bit KV)
template <int KV, int QT, int D, int GB, bool FUSED>
__global__ __launch_bounds__(kWaves * 64) void decode_valu_kernel(StepParams p) {
  const int nx = p.num_q_heads / GB;
  const int seq = blockIdx.x / nx;
  decode_valu_wg<KV, QT, D, GB, FUSED>(p, blockIdx.x - seq * nx, seq, dispatch_part(p));
}

// Merge the partitions of every (row, query head) whose context was split.
// A row of a prefill chunk sees keys 0..its position, split by the chunk
// kernel's partition size; a decode row sees the whole context.  A workgroup
// takes HPW heads of one row, one wave each: in steps with prefill chunks,
// whose rows mostly have nothing to merge, kMultiReduceHeads per workgroup cut
// the workgroups that only check and leave; decode steps keep one head per
// workgroup.  grid.x = head group (fastest), then row.
constexpr int kMultiReduceHeads = 4;
// One wave: query head h of row `row`, partials of type E (float32, or
// bfloat16 for fp8 KV).  Every load that does not need the row's length is
// issued first, so the wave waits on memory about once: this wave's piece of
// the step's append, the (max, sum) of partitions 0..63 (lane q holds
// partition q's; every row owns max_parts entries, read whether written or
// not and masked once the length is known), with AHEAD (decode steps) the
// rows of partitions 0..3, and on steps whose new key is merged here that key's
// score and value.
template <int QT, int D, typename E, bool AHEAD>
__device__ __forceinline__ void reduce_wave(const StepParams& p, int row, int h, int lane) {
  constexpr int C = D / 64;
  constexpr int kAhead = 4;
  constexpr bool FP8 = sizeof(E) == 2;   // bfloat16 partials exactly when the KV is fp8
  const int G = p.num_q_heads / p.num_kv_heads;
  const int kvh = h / G;
  const size_t rh = (size_t)row * p.num_q_heads + h;
  // the step's append when the decode launch read no new row from the pool:
  // the wave of each kv head's first query head stores the row (last)
  const bool appends = p.append_in_merge && h % G == 0;
  U32x4 app{0, 0, 0, 0};
  if (appends) app = load_appended_piece<FP8 ? D : 2 * D>(p, row, kvh, lane);
  const float* ml = p.part_ml + rh * p.max_parts * 2;
  float2 ml0 = make_float2(-__builtin_inff(), 0.f);
  if (lane < p.max_parts) ml0 = *reinterpret_cast<const float2*>(ml + 2 * lane);
  const E* po = reinterpret_cast<const E*>(p.part_o) + rh * p.max_parts * D + lane;
  // (decode steps only: steps with prefill chunks have many rows with
  // nothing to merge.  The reduce runs only where max_parts > 1; past
  // max_parts the last partition is read again and not used.)
  const int ahead = AHEAD ? (p.max_parts < kAhead ? p.max_parts : kAhead) : 0;
  E x0[kAhead][C];
#pragma unroll
  for (int u = 0; u < kAhead; ++u) {
    const int q = u < ahead ? u : ahead - 1;
#pragma unroll
    for (int c = 0; c < C; ++c) x0[u][c] = AHEAD ? po[(size_t)q * D + c * 64] : E(0);
  }
  // the row's length and partition size
  bool merge = true;
  int L = 0, pt = 1, ph = 0;
  if (p.row_seq != nullptr) {
    const int seq = const_load(p.row_seq + row);
    if ((unsigned)seq < (unsigned)p.num_seqs) {
      const int qlen = const_load(p.q_lens + seq);
      L = const_load(p.ctx_lens + seq) - qlen + (row - const_load(p.q_start + seq)) + 1;
      pt = qlen > p.small_q ? p.chunk_part_tokens : p.part_tokens;
      ph = qlen > p.small_q ? 0 : p.part_head;
    } else {
      merge = false;
    }
  } else {
    L = const_load(p.ctx_lens + row);
    pt = p.part_tokens;
    ph = p.part_head;
  }
  // new_in_merge: the partitions cover keys 0 .. L-2 (none when L is 1) and
  // key L-1 is this row's new K/V, merged here as one more partition
  const bool add_new = p.new_in_merge != 0;
  float s_new = 0.f, v_new[C];
  if (add_new) {
    // score of the new key (log2 units, as the partitions' maxima) and its
    // value, dequantised with the scales of the block the row goes to (the
    // scales apply to the sum and to the weight, so their loads, after the
    // slot's, overlap the row's)
    const int slot = const_load(p.slots + row);
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + rh * D;
    const size_t nrow = (size_t)row * p.num_kv_heads + kvh;
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int d = c * 64 + lane;
      const uint16_t qb = qrow[d];
      const float qv = QT == kBF16 ? __uint_as_float((uint32_t)qb << 16)
                                   : (float)__builtin_bit_cast(_Float16, qb);
      float kv, vv, unused;
      if constexpr (FP8) {
        fp8x2_to_f32<false>(p.k_new[nrow * D + d], kv, unused);
        fp8x2_to_f32<false>(p.v_new[nrow * D + d], vv, unused);
      } else {
        const uint16_t kb = reinterpret_cast<const uint16_t*>(p.k_new)[nrow * D + d];
        const uint16_t vb = reinterpret_cast<const uint16_t*>(p.v_new)[nrow * D + d];
        kv = QT == kBF16 ? __uint_as_float((uint32_t)kb << 16) : (float)__builtin_bit_cast(_Float16, kb);
        vv = QT == kBF16 ? __uint_as_float((uint32_t)vb << 16) : (float)__builtin_bit_cast(_Float16, vb);
      }
      dot = __builtin_fmaf(qv, kv, dot);
      v_new[c] = vv;
    }
    float ksc = 1.f, vsc = 1.f;
    if constexpr (FP8) {
      if (slot >= 0 && (int64_t)slot < (int64_t)p.num_blocks * 16) {
        const size_t sc = (size_t)(slot >> 4) * p.num_kv_heads + kvh;
        ksc = p.k_scale[sc];
        vsc = p.v_scale[sc];
      }
    }
    s_new = wave_sum(dot) * ksc * p.scale_log2;
#pragma unroll
    for (int c = 0; c < C; ++c) v_new[c] *= vsc;
  }
  if (L < 1 || L > p.max_blocks * 16 || L + ph > p.max_parts * pt) merge = false;
  const int nparts = merge ? part_count(add_new ? L - 1 : L, pt, ph) : 0;
  if (nparts <= 1 && !add_new) merge = false;
  if (merge) {
    const float m_first = lane < nparts ? ml0.x : -__builtin_inff();
    const float l_first = lane < nparts ? ml0.y : 0.f;
    float M = m_first;
    for (int q = lane + 64; q < nparts; q += 64) M = fmaxf(M, ml[2 * q]);
    M = wave_max(M);
    if (add_new) M = fmaxf(M, s_new);
    float ls = 0.f;
    float o[C];
#pragma unroll
    for (int c = 0; c < C; ++c) o[c] = 0.f;
    // partitions are added in index order, 64 at a time: lane j holds the
    // weight of partition base + j, read back with readlane, and the rows of
    // four partitions are loaded together
    for (int base = 0; base < nparts; base += 64) {
      float mq = m_first, lq = l_first;
      if (base > 0) {
        const int q = base + lane;
        mq = q < nparts ? ml[2 * q] : -__builtin_inff();
        lq = q < nparts ? ml[2 * q + 1] : 0.f;
      }
      const float fq = __builtin_amdgcn_exp2f(mq - M);
      const int n = nparts - base < 64 ? nparts - base : 64;
      auto add = [&](int j, const E* x) {
        const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fq), j));
        const float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lq), j));
        ls = __builtin_fmaf(l, f, ls);
#pragma unroll
        for (int c = 0; c < C; ++c) {
          float v;
          if constexpr (sizeof(E) == 2) v = __uint_as_float((uint32_t)x[c] << 16);
          else v = x[c];
          o[c] = __builtin_fmaf(v, f, o[c]);
        }
      };
      const E* pb = po + (size_t)base * D;
      int j = 0;
      if (base == 0) {
#pragma unroll
        for (int u = 0; u < kAhead; ++u)
          if (u < ahead && u < n) add(u, x0[u]);
        j = ahead < n ? ahead : n;
      }
      for (; j + 4 <= n; j += 4) {
        E x[4][C];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int c = 0; c < C; ++c) x[u][c] = pb[(size_t)(j + u) * D + c * 64];
#pragma unroll
        for (int u = 0; u < 4; ++u) add(j + u, x[u]);
      }
      for (; j < n; ++j) {
        E x[C];
#pragma unroll
        for (int c = 0; c < C; ++c) x[c] = pb[(size_t)j * D + c * 64];
        add(j, x);
      }
    }
    if (add_new) {
      const float f = __builtin_amdgcn_exp2f(s_new - M);
      ls += f;
#pragma unroll
      for (int c = 0; c < C; ++c) o[c] = __builtin_fmaf(v_new[c], f, o[c]);
    }
#pragma unroll
    for (int c = 0; c < C; ++c)
      reinterpret_cast<uint16_t*>(p.out)[rh * D + c * 64 + lane] = to_out_bits<QT>(o[c] / ls);
  }
  if (appends) store_appended_piece<FP8 ? D : 2 * D>(p, row, kvh, lane, app);
}

// E: the partials' type (bfloat16 for fp8 KV, else float32), one kernel each
template <int QT, int D, int HPW, typename E>
__global__ __launch_bounds__(64 * HPW) void split_reduce_kernel(StepParams p) {
  const int ng = (p.num_q_heads + HPW - 1) / HPW;
  const int row = blockIdx.x / ng;
  const int h = (blockIdx.x - row * ng) * HPW + (HPW > 1 ? (int)(threadIdx.x >> 6) : 0);
  const int lane = threadIdx.x & 63;
  if (h >= p.num_q_heads) return;
  // one head per workgroup on decode steps, which read partitions ahead
  reduce_wave<QT, D, E, HPW == 1>(p, row, h, lane);
}

// inclusive scan of v over the 1024 threads of the workgroup
__device__ __forceinline__ int block_scan_1024(int v, int32_t* wave_tot) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  for (int w = 0; w < wave; ++w) x += wave_tot[w];
  __syncthreads();
  return x;
}

// Row offsets of every sequence (exclusive scan of query_lens), the owning
// sequence of every query row, and the list of (sequence, first column)
// entries of chunk_cols (row, head) columns of every sequence with more than small_q
// query rows (shorter ones, e.g. speculative-decoding verify rows, run as
// decode items).
// One workgroup; only launched when some sequence has more than one row.
// Workgroups 1 .. append_rows (16-bit KV with the step's append in this
// launch) each store one row's new K and V into its slot first, as the append
// kernel does: the step kernel after this launch reads them from the pool.
__global__ __launch_bounds__(1024) void step_prologue_kernel(StepParams p) {
  if (blockIdx.x > 0) {
    const int row = blockIdx.x - 1;
    const int slot = p.slots[row];
    if (slot < 0 || (int64_t)slot >= (int64_t)p.num_blocks * 16) return;
    const int rb = p.append_row_bytes;
    const int pph = rb / 16;                                 // 16-byte pieces per (row, head)
    const int per = p.num_kv_heads * pph;                    // pieces of K (then of V)
    const size_t base = (size_t)row * p.num_kv_heads * rb;
    const size_t blk = (size_t)(slot >> 4), off = (size_t)(slot & 15);
    for (int j = threadIdx.x; j < 2 * per; j += blockDim.x) {
      const bool is_v = j >= per;
      const int jj = j - (is_v ? per : 0);
      const int head = jj / pph;
      const int piece = jj - head * pph;
      const uint4 x = *reinterpret_cast<const uint4*>((is_v ? p.v_new : p.k_new) + base + (size_t)jj * 16);
      *reinterpret_cast<uint4*>(const_cast<uint8_t*>(is_v ? p.v_pool : p.k_pool) +
                                ((blk * p.num_kv_heads + head) * 16 + off) * rb + (size_t)piece * 16) = x;
    }
    return;
  }
  constexpr int kBig = 256;                 // long sequences filled by the whole workgroup
  __shared__ int32_t wave_tot[16];
  __shared__ int32_t carry_rows, carry_tiles, n_big;
  __shared__ int32_t big_seq[kBig], big_start[kBig], big_q[kBig], big_tstart[kBig], big_tiles[kBig];
  int32_t* q_start = const_cast<int32_t*>(p.q_start);
  int32_t* row_seq = const_cast<int32_t*>(p.row_seq);
  int32_t* entries = const_cast<int32_t*>(p.chunk_entries);
  const int group = p.num_q_heads / p.num_kv_heads;
  const int tid = threadIdx.x;
  if (tid == 0) { carry_rows = 0; carry_tiles = 0; n_big = 0; }
  __syncthreads();
  for (int base = 0; base < p.num_seqs; base += 1024) {
    const int i = base + tid;
    const int q = i < p.num_seqs ? max(p.q_lens[i], 0) : 0;
    const int cc = p.chunk_cols;
    const int tiles = q > p.small_q ? (q * group + cc - 1) / cc : 0;   // chunk entries
    const int r_incl = block_scan_1024(q, wave_tot);
    const int t_incl = block_scan_1024(tiles, wave_tot);
    const int start = carry_rows + r_incl - q;
    const int tstart = carry_tiles + t_incl - tiles;
    bool serial = true;
    if (i < p.num_seqs) {
      q_start[i] = start;
      if (q > 32 || tiles > 8) {
        const int k = atomicAdd(&n_big, 1);
        if (k < kBig) {
          big_seq[k] = i; big_start[k] = start; big_q[k] = q;
          big_tstart[k] = tstart; big_tiles[k] = tiles;
          serial = false;
        }
      }
      if (serial) {
        const int stop = min(start + q, p.total_q);
        for (int r = max(start, 0); r < stop; ++r) row_seq[r] = i;
        for (int t = 0; t < tiles && tstart + t < p.chunk_capacity; ++t) {
          entries[2 * (tstart + t)] = i;
          entries[2 * (tstart + t) + 1] = cc * t;
        }
      }
    }
    __syncthreads();
    const int nb = min(n_big, kBig);
    for (int k = 0; k < nb; ++k) {
      const int st = big_start[k];
      for (int r = tid; r < big_q[k]; r += 1024)
        if (st + r >= 0 && st + r < p.total_q) row_seq[st + r] = big_seq[k];
      for (int t = tid; t < big_tiles[k]; t += 1024)
        if (big_tstart[k] + t < p.chunk_capacity) {
          entries[2 * (big_tstart[k] + t)] = big_seq[k];
          entries[2 * (big_tstart[k] + t) + 1] = p.chunk_cols * t;
        }
    }
    __syncthreads();
    if (tid == 1023) { carry_rows += r_incl; carry_tiles += t_incl; }
    if (tid == 0) n_big = 0;
    __syncthreads();
  }
  if (tid == 0) {
    q_start[p.num_seqs] = carry_rows;
    *const_cast<int32_t*>(p.chunk_count) = min(carry_tiles, p.chunk_capacity);
  }
}

// ---------------------------------------------------------------------------
// contract checks (launched by the checks build only)
// ---------------------------------------------------------------------------
// The device-resident metadata of a step against the contract of
// paged_attn_step (page "Serving LLMs with vLLM", sections "Blocks and Block
// Tables" and "Attention Over Scattered Blocks": every table entry a context
// reaches names a block of the pool; a context fits its table; query rows sit
// at the end of their context).  One workgroup clears the record, then reads
// every length and every table entry a context reaches; the first violation
// it meets (in no particular order) is recorded with its sequence, index and
// value, and all are counted.  It only reads metadata, never the pools.
// rec: [0] code, [1] sequence, [2] index (table column; -1 for lengths),
// [3] offending value, [4] number of violations.
__global__ __launch_bounds__(1024) void step_check_kernel(StepParams p, int32_t* rec,
                                                          int32_t max_ctx, int32_t max_q) {
  __shared__ int32_t rows;
  const int tid = threadIdx.x;
  if (tid == 0) {
    rec[0] = kViolationNone;
    rec[1] = -1;
    rec[2] = -1;
    rec[3] = 0;
    rec[4] = 0;
    rows = 0;
  }
  __syncthreads();
  auto flag = [&](int code, int seq, int index, int value) {
    atomicAdd(&rec[4], 1);
    if (atomicCAS(&rec[0], kViolationNone, code) == kViolationNone) {
      rec[1] = seq;
      rec[2] = index;
      rec[3] = value;
    }
  };
  const int table_cap = p.max_blocks * 16;
  for (int i = tid; i < p.num_seqs; i += blockDim.x) {
    const int L = p.ctx_lens[i];
    const int Q = p.q_lens[i];
    atomicAdd(&rows, Q);
    if (L < 1 || L > table_cap || L > max_ctx) flag(kViolationContextLen, i, -1, L);
    else if (Q < 1 || Q > L || Q > max_q) flag(kViolationQueryLen, i, -1, Q);
  }
  const long long entries = (long long)p.num_seqs * p.max_blocks;
  for (long long e = tid; e < entries; e += blockDim.x) {
    const int i = (int)(e / p.max_blocks);
    const int j = (int)(e - (long long)i * p.max_blocks);
    const int L = p.ctx_lens[i];
    if (L < 1 || L > table_cap || j >= (L + 15) / 16) continue;
    const int b = p.tables[e];
    if (b < 0 || b >= p.num_blocks) flag(kViolationBlockId, i, j, b);
  }
  __syncthreads();
  if (tid == 0 && rows != p.total_q) flag(kViolationTotalRows, -1, -1, rows);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_check(const StepParams& p, int32_t* record, int32_t max_ctx, int32_t max_q,
                        hipStream_t stream) {
  (void)hipGetLastError();   // drop an error some earlier, unrelated call left behind
  hipLaunchKernelGGL(step_check_kernel, dim3(1), dim3(1024), 0, stream, p, record, max_ctx, max_q);
  return hipGetLastError();
}

hipError_t launch_prologue(const StepParams& p, hipStream_t stream) {
  (void)hipGetLastError();   // drop an error some earlier, unrelated call left behind
  hipLaunchKernelGGL(step_prologue_kernel, dim3(1 + (uint32_t)p.append_rows), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

template <int KV, int QT, int D>
static hipError_t decode_by_group(const StepParams& p, const StepPlan& plan, hipStream_t stream) {
  const dim3 grid((uint32_t)(p.num_q_heads / plan.heads_per_wg * p.num_seqs), (uint32_t)p.max_parts);
  const dim3 block(kWaves * 64);
  (void)hipGetLastError();   // drop an error some earlier, unrelated call left behind
  if (p.k_new != nullptr) {
    // the append in this launch: 16-bit KV, one or two query heads per kv head
    if constexpr (KV == kFP8) return hipErrorInvalidValue;
    else switch (plan.heads_per_wg) {
      case 1: hipLaunchKernelGGL((decode_valu_kernel<KV, QT, D, 1, true>), grid, block, 0, stream, p); break;
      case 2: hipLaunchKernelGGL((decode_valu_kernel<KV, QT, D, 2, true>), grid, block, 0, stream, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (plan.heads_per_wg) {
    case 1: hipLaunchKernelGGL((decode_valu_kernel<KV, QT, D, 1, false>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_valu_kernel<KV, QT, D, 2, false>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_valu_kernel<KV, QT, D, 4, false>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_valu_kernel<KV, QT, D, 8, false>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KV, int QT>
static hipError_t decode_by_dim(const StepParams& p, const StepPlan& plan, hipStream_t stream) {
  if (plan.head_dim == 128) return decode_by_group<KV, QT, 128>(p, plan, stream);
  if (plan.head_dim == 64) return decode_by_group<KV, QT, 64>(p, plan, stream);
  return hipErrorInvalidValue;
}

bool decode_supported(const StepPlan& plan) {
  const bool dim_ok = plan.head_dim == 64 || plan.head_dim == 128;
  const bool gb_ok = plan.heads_per_wg == 1 || plan.heads_per_wg == 2 || plan.heads_per_wg == 4 ||
                     plan.heads_per_wg == 8;
  const bool q_ok = plan.q_dtype == kF16 || plan.q_dtype == kBF16;
  const bool kv_ok = plan.kv_dtype == plan.q_dtype || plan.kv_dtype == kFP8;
  return dim_ok && gb_ok && q_ok && kv_ok;
}

hipError_t launch_decode(const StepParams& p, const StepPlan& plan, hipStream_t stream) {
  if (plan.q_dtype == kBF16) {
    if (plan.kv_dtype == kBF16) return decode_by_dim<kBF16, kBF16>(p, plan, stream);
    if (plan.kv_dtype == kFP8) return decode_by_dim<kFP8, kBF16>(p, plan, stream);
  } else if (plan.q_dtype == kF16) {
    if (plan.kv_dtype == kF16) return decode_by_dim<kF16, kF16>(p, plan, stream);
    if (plan.kv_dtype == kFP8) return decode_by_dim<kFP8, kF16>(p, plan, stream);
  }
  return hipErrorInvalidValue;
}

template <int HPW, typename E>
void reduce_launch(const StepParams& p, const StepPlan& plan, dim3 grid, dim3 block, hipStream_t stream) {
  if (plan.q_dtype == kBF16) {
    if (plan.head_dim == 128) hipLaunchKernelGGL((split_reduce_kernel<kBF16, 128, HPW, E>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((split_reduce_kernel<kBF16, 64, HPW, E>), grid, block, 0, stream, p);
  } else {
    if (plan.head_dim == 128) hipLaunchKernelGGL((split_reduce_kernel<kF16, 128, HPW, E>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((split_reduce_kernel<kF16, 64, HPW, E>), grid, block, 0, stream, p);
  }
}

template <int HPW>
void reduce_typed(const StepParams& p, const StepPlan& plan, dim3 grid, hipStream_t stream) {
  const dim3 block(64 * HPW);
  if (p.part_bf16) reduce_launch<HPW, uint16_t>(p, plan, grid, block, stream);
  else reduce_launch<HPW, float>(p, plan, grid, block, stream);
}

hipError_t launch_reduce(const StepParams& p, const StepPlan& plan, hipStream_t stream) {
  (void)hipGetLastError();   // drop an error some earlier, unrelated call left behind
  if (p.row_seq != nullptr) {
    constexpr int H = kMultiReduceHeads;
    const dim3 grid((uint32_t)((p.num_q_heads + H - 1) / H * p.total_q));
    reduce_typed<H>(p, plan, grid, stream);
  } else {
    reduce_typed<1>(p, plan, dim3((uint32_t)(p.num_q_heads * p.total_q)), stream);
  }
  return hipGetLastError();
}

}  // namespace pkv
