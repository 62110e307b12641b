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
//   grid.x  group of `GB` query heads that share one kv head,
//   grid.y  sequence (only sequences with one query row; prefill chunks go to
//           the MFMA chunk kernel),
//   grid.z  split-context partition of part_tokens tokens.
// The hardware deals workgroups to the 8 XCDs round-robin by linear id, so the
// fastest grid dimension must not be one along which the work per workgroup
// changes: heads (equal work) go first and partitions (the last ones are often
// empty) go last, which also dispatches every row's heavy first partitions
// before the light tail ones.
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

#include "pkv_launch.h"

namespace pkv {

constexpr int kWaves = 4;

// Shape constants of the register layout for one (KV type, head_dim).
template <int KV, int D>
struct Lay {
  static constexpr int ELT = (KV == kFP8) ? 1 : 2;   // bytes per KV element
  static constexpr int ROWB = D * ELT;                // bytes of one token row of one head
  static constexpr int LPR = ROWB / 16;               // lanes per token row
  static constexpr int RPL = 64 / LPR;                // token rows per wave-wide load
  static constexpr int NL = 16 / RPL;                 // loads per 16-token block
  static constexpr int EPL = 16 / ELT;                // elements per lane per load
  static constexpr int BLKB = 16 * ROWB;              // bytes of one (block, head)
  // 16-bit K is multiplied pairwise with v_dot2 against 16-bit q; fp8 K goes through fp32
  static constexpr bool DOT2 = KV != kFP8;
};

// Scores, online-softmax update and value accumulation for one 16-token block.
// kr / vr hold this lane's slice of the block's K and V rows; `limit` is the
// number of the block's tokens that belong to the sequence (16 for all but the
// last block; 0 for a block whose table entry is out of range).
template <int KV, int QT, int D, int GB>
__device__ __forceinline__ void attend_block(const uint4 (&kr)[Lay<KV, D>::NL],
                                             const uint4 (&vr)[Lay<KV, D>::NL], float ksc,
                                             float vsc, int limit, int rg,
                                             const uint32_t (&qp)[GB][Lay<KV, D>::EPL / 2],
                                             const float (&qf)[GB][Lay<KV, D>::EPL],
                                             float score_mul, float (&m)[GB], float (&l)[GB],
                                             float (&acc)[GB][Lay<KV, D>::EPL]) {
  using T = Lay<KV, D>;
  float s[GB][T::NL];
#pragma unroll
  for (int j = 0; j < T::NL; ++j) {
    if constexpr (T::DOT2) {
      const uint32_t w[4] = {kr[j].x, kr[j].y, kr[j].z, kr[j].w};
#pragma unroll
      for (int g = 0; g < GB; ++g) {
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if constexpr (KV == kBF16)
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qp[g][c]),
                                                __builtin_bit_cast(bf16x2, w[c]), a, false);
          else
            a = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, qp[g][c]),
                                       __builtin_bit_cast(f16x2, w[c]), a, false);
        }
        s[g][j] = group_sum<T::LPR>(a) * score_mul;
      }
    } else {
      float kf[T::EPL];
      unpack16<KV>(kr[j], kf);
#pragma unroll
      for (int g = 0; g < GB; ++g) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < T::EPL; ++e) a = __builtin_fmaf(qf[g][e], kf[e], a);
        s[g][j] = group_sum<T::LPR>(a) * ksc;
      }
    }
  }

  const bool full = limit >= 16;
  bool valid[T::NL];
#pragma unroll
  for (int j = 0; j < T::NL; ++j) valid[j] = full || (j * T::RPL + rg < limit);

  float pw[GB][T::NL];
#pragma unroll
  for (int g = 0; g < GB; ++g) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < T::NL; ++j) mx = fmaxf(mx, valid[j] ? s[g][j] : -__builtin_inff());
    const float mn = fmaxf(m[g], mx);
    const float alpha = __builtin_amdgcn_exp2f(m[g] - mn);
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < T::NL; ++j) {
      pw[g][j] = valid[j] ? __builtin_amdgcn_exp2f(s[g][j] - mn) : 0.f;
      ps += pw[g][j];
    }
    l[g] = l[g] * alpha + ps;
    m[g] = mn;
    if (__any(alpha != 1.f)) {       // the running max rarely moves after the first blocks
#pragma unroll
      for (int e = 0; e < T::EPL; ++e) acc[g][e] *= alpha;
    }
  }

#pragma unroll
  for (int j = 0; j < T::NL; ++j) {
    float vf[T::EPL];
    unpack16<KV>(vr[j], vf);
    if (!full) {
#pragma unroll
      for (int e = 0; e < T::EPL; ++e) vf[e] = valid[j] ? vf[e] : 0.f;   // select: tail slots may hold NaN
    }
#pragma unroll
    for (int g = 0; g < GB; ++g) {
      const float pv = pw[g][j] * vsc;
#pragma unroll
      for (int e = 0; e < T::EPL; ++e) acc[g][e] = __builtin_fmaf(pv, vf[e], acc[g][e]);
    }
  }
}

template <int KV, int QT, int D, int GB>
__global__ __launch_bounds__(kWaves * 64) void decode_valu_kernel(StepParams p) {
  using T = Lay<KV, D>;
  static_assert(T::LPR >= 1 && T::LPR <= 16 && T::NL >= 1, "unsupported shape");
  static_assert(!T::DOT2 || KV == QT, "16-bit KV is read with q of the same type");

  const int part = blockIdx.z;
  const int seq = blockIdx.y;
  const int lane = threadIdx.x & 63;
  // wave-uniform by construction; readfirstlane lets the compiler keep what derives
  // from it (block indices, buffer resources) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = p.num_q_heads / p.num_kv_heads;
  const int h0 = blockIdx.x * GB;                // first query head of this workgroup
  const int kvh = h0 / group;

  int row = seq;
  if (p.q_start != nullptr) {
    if (p.q_lens[seq] != 1) return;              // prefill chunks go to the chunk kernel
    row = p.q_start[seq];
    if (row < 0 || row >= p.total_q) return;
  }
  const int L = p.ctx_lens[seq];
  const int tok0 = part * p.part_tokens;
  // rows whose length breaks the host scalars' promises are left unwritten
  if (tok0 >= L || L > p.max_blocks * 16 || L > p.max_parts * p.part_tokens) return;
  const int nparts = (L + p.part_tokens - 1) / p.part_tokens;
  const int blk_begin = tok0 >> 4;
  const int blk_end = min((L + 15) >> 4, (tok0 + p.part_tokens) >> 4);

  // block table entries of this wave's blocks (blk_begin + wave + kWaves * i)
  const int32_t* trow = p.tables + (size_t)seq * p.max_blocks;
  const int nb = blk_end - blk_begin;
  const int cnt = nb > wave ? (nb - wave + kWaves - 1) / kWaves : 0;   // <= 64 by construction
  const int my_tbl = lane < cnt ? trow[blk_begin + wave + kWaves * lane] : -1;
  // fp8 scales of the same blocks, one per lane (read per block with readlane)
  float my_ks = 1.f, my_vs = 1.f;
  if constexpr (KV == kFP8) {
    if ((unsigned)my_tbl < (unsigned)p.num_blocks) {
      my_ks = p.k_scale[(size_t)my_tbl * p.num_kv_heads + kvh];
      my_vs = p.v_scale[(size_t)my_tbl * p.num_kv_heads + kvh];
    }
  }

  // this lane's slice of the GB query vectors: raw 16-bit pairs for the dot2
  // path (the score is scaled afterwards), fp32 pre-scaled into log2 units otherwise
  const int dim0 = (lane % T::LPR) * T::EPL;
  uint32_t qp[GB][T::EPL / 2];
  float qf[GB][T::EPL];
#pragma unroll
  for (int g = 0; g < GB; ++g) {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           ((size_t)row * p.num_q_heads + h0 + g) * D + dim0;
#pragma unroll
    for (int c = 0; c < T::EPL / 8; ++c) {
      const uint4 r = reinterpret_cast<const uint4*>(qrow)[c];
      if constexpr (T::DOT2) {
        qp[g][4 * c + 0] = r.x;
        qp[g][4 * c + 1] = r.y;
        qp[g][4 * c + 2] = r.z;
        qp[g][4 * c + 3] = r.w;
      } else {
        float f[8];
        if constexpr (QT == kBF16) unpack16<kBF16>(r, f);
        else unpack16<kF16>(r, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[g][c * 8 + e] = f[e] * p.scale_log2;
      }
    }
  }

  float m[GB], l[GB], acc[GB][T::EPL];
#pragma unroll
  for (int g = 0; g < GB; ++g) {
    m[g] = kMaxSeed;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < T::EPL; ++e) acc[g][e] = 0.f;
  }

  const int rg = lane / T::LPR;                  // token row group of this lane
  // Two register buffers: the loads of block i+1 are in flight while block i is
  // scored.  Every iteration issues the same loads with no branch around them
  // (past the phase's last block the index is clamped and the block counts no
  // tokens), so the compiler can wait for exactly the block it needs instead of
  // draining every outstanding load at a control-flow join.  An out-of-range
  // table entry reads block 0 and counts no tokens.
  uint4 kA[T::NL], vA[T::NL], kB[T::NL], vB[T::NL];
  float kscA = 1.f, vscA = 1.f, kscB = 1.f, vscB = 1.f;
  int limA = 0, limB = 0;
  auto issue = [&](auto nt, int i, int end, uint4 (&kr)[T::NL], uint4 (&vr)[T::NL], float& ks,
                   float& vs, int& lim) {
    constexpr bool NT = decltype(nt)::value;
    const int ic = min(i, end - 1);
    const int b = blk_begin + wave + kWaves * ic;
    int phys = __builtin_amdgcn_readlane(my_tbl, ic);
    lim = i < end ? min(16, L - b * 16) : 0;
    if ((unsigned)phys >= (unsigned)p.num_blocks) { phys = 0; lim = 0; }
    const size_t boff = ((size_t)phys * p.num_kv_heads + kvh) * T::BLKB;
    // a block with no tokens is not read (the count kept scalar: no waterfall loop)
    const int bytes = __builtin_amdgcn_readfirstlane(lim > 0 ? T::BLKB : 0);
    const __amdgpu_buffer_rsrc_t kres = block_rsrc(p.k_pool + boff, bytes);
    const __amdgpu_buffer_rsrc_t vres = block_rsrc(p.v_pool + boff, bytes);
#pragma unroll
    for (int j = 0; j < T::NL; ++j) kr[j] = load_block16<NT>(kres, (j * 64 + lane) * 16);
#pragma unroll
    for (int j = 0; j < T::NL; ++j) vr[j] = load_block16<NT>(vres, (j * 64 + lane) * 16);
    if constexpr (KV == kFP8) {
      ks = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_ks), ic));
      vs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_vs), ic));
    }
  };
  // blocks i0 .. i1-1 of this wave, with one load policy
  auto walk = [&](auto nt, int i0, int i1) {
    if (i1 <= i0) return;
    issue(nt, i0, i1, kA, vA, kscA, vscA, limA);
    for (int i = i0; i < i1; i += 2) {
      issue(nt, i + 1, i1, kB, vB, kscB, vscB, limB);
      attend_block<KV, QT, D, GB>(kA, vA, kscA, vscA, limA, rg, qp, qf, p.scale_log2, m, l, acc);
      issue(nt, i + 2, i1, kA, vA, kscA, vscA, limA);
      attend_block<KV, QT, D, GB>(kB, vB, kscB, vscB, limB, rg, qp, qf, p.scale_log2, m, l, acc);
    }
  };
  // blocks other sequences also read stay cacheable; the rest stream past the
  // caches.  The hint is clamped to this partition's blocks first, so no value
  // of it can overflow the arithmetic below: 0 <= cnt_sh <= cnt.
  const int hint = p.shared_blocks != nullptr ? p.shared_blocks[seq] : 0;
  const int nsh = min(max(hint, blk_begin), blk_end);
  const int cnt_sh = min(cnt, max(0, nsh - blk_begin - wave + kWaves - 1) / kWaves);
  walk(std::false_type{}, 0, cnt_sh);
  walk(std::true_type{}, cnt_sh, cnt);

  // merge the RPL token-row groups of this wave
#pragma unroll
  for (int g = 0; g < GB; ++g) {
    float M = m[g];
#pragma unroll
    for (int off = T::LPR; off < 64; off <<= 1) M = fmaxf(M, shfl_xor_f(M, off));
    const float f = __builtin_amdgcn_exp2f(m[g] - M);
    l[g] *= f;
#pragma unroll
    for (int e = 0; e < T::EPL; ++e) acc[g][e] *= f;
#pragma unroll
    for (int off = T::LPR; off < 64; off <<= 1) {
      l[g] += shfl_xor_f(l[g], off);
#pragma unroll
      for (int e = 0; e < T::EPL; ++e) acc[g][e] += shfl_xor_f(acc[g][e], off);
    }
    m[g] = M;
  }

  // merge the waves through LDS
  __shared__ float sm_o[kWaves][GB][D];
  __shared__ float sm_m[kWaves][GB];
  __shared__ float sm_l[kWaves][GB];
  if (rg == 0) {
#pragma unroll
    for (int g = 0; g < GB; ++g)
#pragma unroll
      for (int e = 0; e < T::EPL; ++e) sm_o[wave][g][dim0 + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GB; ++g) { sm_m[wave][g] = m[g]; sm_l[wave][g] = l[g]; }
  }
  __syncthreads();

  for (int t = threadIdx.x; t < GB * D; t += kWaves * 64) {
    const int g = t / D;
    const int d = t - g * D;
    float M = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][g]);
    float ls = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm_m[w][g] - M);
      ls = __builtin_fmaf(sm_l[w][g], f, ls);
      o = __builtin_fmaf(sm_o[w][g][d], f, o);
    }
    const size_t rh = (size_t)row * p.num_q_heads + h0 + g;
    if (nparts == 1) {
      reinterpret_cast<uint16_t*>(p.out)[rh * D + d] = to_out_bits<QT>(o / ls);
    } else {
      const size_t idx = rh * p.max_parts + part;
      p.part_o[idx * D + d] = o;
      if (d == 0) {
        p.part_ml[idx * 2] = M;
        p.part_ml[idx * 2 + 1] = ls;
      }
    }
  }
}

// Merge the partitions of every (row, query head) whose context was split.
// A row of a prefill chunk sees keys 0..its position, split by the chunk
// kernel's partition size; a decode row sees the whole context.  A workgroup
// takes HPW heads of one row, one wave each: in steps with prefill chunks,
// whose rows mostly have nothing to merge, kMultiReduceHeads per workgroup cut
// the workgroups that only check and leave; decode steps keep one head per
// workgroup.
constexpr int kMultiReduceHeads = 4;
template <int QT, int D, int HPW>
__global__ __launch_bounds__(64 * HPW) void split_reduce_kernel(StepParams p) {
  const int h = blockIdx.x * HPW + (HPW > 1 ? (int)(threadIdx.x >> 6) : 0);
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.y;
  if (h >= p.num_q_heads) return;
  int L, pt;
  if (p.row_seq != nullptr) {
    const int seq = p.row_seq[row];
    if ((unsigned)seq >= (unsigned)p.num_seqs) return;
    const int qlen = p.q_lens[seq];
    L = p.ctx_lens[seq] - qlen + (row - p.q_start[seq]) + 1;
    pt = qlen > p.small_q ? p.chunk_part_tokens : p.part_tokens;
  } else {
    L = p.ctx_lens[row];
    pt = p.part_tokens;
  }
  if (L < 1 || L > p.max_blocks * 16 || L > p.max_parts * pt) return;
  const int nparts = (L + pt - 1) / pt;
  if (nparts <= 1) return;
  const size_t rh = (size_t)row * p.num_q_heads + h;
  const float* ml = p.part_ml + rh * p.max_parts * 2;
  const float* po = p.part_o + rh * p.max_parts * D;
  float M = -__builtin_inff();
  for (int q = 0; q < nparts; ++q) M = fmaxf(M, ml[2 * q]);
  float ls = 0.f;
  float o[D / 64];
#pragma unroll
  for (int c = 0; c < D / 64; ++c) o[c] = 0.f;
  for (int q = 0; q < nparts; ++q) {
    const float f = __builtin_amdgcn_exp2f(ml[2 * q] - M);
    ls = __builtin_fmaf(ml[2 * q + 1], f, ls);
#pragma unroll
    for (int c = 0; c < D / 64; ++c)
      o[c] = __builtin_fmaf(po[(size_t)q * D + c * 64 + lane], f, o[c]);
  }
#pragma unroll
  for (int c = 0; c < D / 64; ++c)
    reinterpret_cast<uint16_t*>(p.out)[rh * D + c * 64 + lane] = to_out_bits<QT>(o[c] / ls);
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
__global__ __launch_bounds__(1024) void step_prologue_kernel(StepParams p) {
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
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_prologue(const StepParams& p, hipStream_t stream) {
  (void)hipGetLastError();   // drop an error some earlier, unrelated call left behind
  hipLaunchKernelGGL(step_prologue_kernel, dim3(1), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

template <int KV, int QT, int D>
static hipError_t decode_by_group(const StepParams& p, const StepPlan& plan, hipStream_t stream) {
  const dim3 grid((uint32_t)(p.num_q_heads / plan.heads_per_wg), (uint32_t)p.num_seqs,
                  (uint32_t)p.max_parts);
  const dim3 block(kWaves * 64);
  (void)hipGetLastError();   // drop an error some earlier, unrelated call left behind
  switch (plan.heads_per_wg) {
    case 1: hipLaunchKernelGGL((decode_valu_kernel<KV, QT, D, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_valu_kernel<KV, QT, D, 2>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_valu_kernel<KV, QT, D, 4>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_valu_kernel<KV, QT, D, 8>), grid, block, 0, stream, p); break;
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

template <int HPW>
void reduce_typed(const StepParams& p, const StepPlan& plan, dim3 grid, hipStream_t stream) {
  const dim3 block(64 * HPW);
  if (plan.q_dtype == kBF16) {
    if (plan.head_dim == 128) hipLaunchKernelGGL((split_reduce_kernel<kBF16, 128, HPW>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((split_reduce_kernel<kBF16, 64, HPW>), grid, block, 0, stream, p);
  } else {
    if (plan.head_dim == 128) hipLaunchKernelGGL((split_reduce_kernel<kF16, 128, HPW>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((split_reduce_kernel<kF16, 64, HPW>), grid, block, 0, stream, p);
  }
}

hipError_t launch_reduce(const StepParams& p, const StepPlan& plan, hipStream_t stream) {
  (void)hipGetLastError();   // drop an error some earlier, unrelated call left behind
  if (p.row_seq != nullptr) {
    constexpr int H = kMultiReduceHeads;
    const dim3 grid((uint32_t)((p.num_q_heads + H - 1) / H), (uint32_t)p.total_q);
    reduce_typed<H>(p, plan, grid, stream);
  } else {
    reduce_typed<1>(p, plan, dim3((uint32_t)p.num_q_heads, (uint32_t)p.total_q), stream);
  }
  return hipGetLastError();
}

}  // namespace pkv
