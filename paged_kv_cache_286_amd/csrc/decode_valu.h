// VALU decode workgroup for gfx950: block-table walk, 16-byte coalesced KV
// loads, fp32 online softmax with DPP reductions, split-context partials.
// Shared by the decode kernel and the step kernel of steps with prefill chunks.
//
// Page "Serving LLMs with vLLM: Continuous Batching and PagedAttention
// Explained", section "Attention Over Scattered Blocks": the kernel reads the
// block table, fetches each block from its physical place and scores block by
// block; the result is ordinary softmax attention over the whole history.
// Section "Blocks and Block Tables" fixes the addressing: token t of a
// sequence sits in block table[t / 16] at offset t % 16.
#pragma once
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

// The row's new K and V (ROWB bytes per (row, kv head)) into its slot for kv
// head kvh: one 16-byte piece per lane, K on the first ROWB/16 lanes, V on the
// next; a slot outside the pool (or -1) stores nothing, as in the append kernel.
template <int ROWB>
__device__ __forceinline__ void store_appended_row(const StepParams& p, int row, int kvh, int lane) {
  constexpr int LPR = ROWB / 16;
  const int slot = p.slots[row];
  if (lane < 2 * LPR && slot >= 0 && (int64_t)slot < (int64_t)p.num_blocks * 16) {
    const bool is_v = lane >= LPR;
    const int piece = lane - (is_v ? LPR : 0);
    const size_t src = ((size_t)row * p.num_kv_heads + kvh) * ROWB + piece * 16;
    const size_t dst =
        (((size_t)(slot >> 4) * p.num_kv_heads + kvh) * 16 + (slot & 15)) * ROWB + piece * 16;
    const uint4 x = *reinterpret_cast<const uint4*>((is_v ? p.v_new : p.k_new) + src);
    *reinterpret_cast<uint4*>(const_cast<uint8_t*>(is_v ? p.v_pool : p.k_pool) + dst) = x;
  }
}

// The same piece in two halves, so that other loads can go between them:
// load_appended_piece reads the lane's piece of the new row (whatever the
// slot: the step's new rows all exist), store_appended_piece writes it to the
// row's slot.  The pointers are taken into scalar registers and accessed as
// global memory: a per-lane choice between two kernel arguments otherwise
// becomes a vector load of the chosen pointer, and a flat access would also
// hold back every later wait on scalar loads.
typedef uint32_t U32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) U32x4 GlobalU32x4;
__device__ __forceinline__ GlobalU32x4* global_uniform(const void* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (GlobalU32x4*)(((uint64_t)hi << 32) | lo);
}
template <int ROWB>
__device__ __forceinline__ U32x4 load_appended_piece(const StepParams& p, int row, int kvh, int lane) {
  constexpr int LPR = ROWB / 16;
  U32x4 x{0, 0, 0, 0};
  GlobalU32x4* src_k = global_uniform(p.k_new);
  GlobalU32x4* src_v = global_uniform(p.v_new);
  if (lane < 2 * LPR) {
    const bool is_v = lane >= LPR;
    const int piece = lane - (is_v ? LPR : 0);
    x = (is_v ? src_v : src_k)[((size_t)row * p.num_kv_heads + kvh) * LPR + piece];
  }
  return x;
}
template <int ROWB>
__device__ __forceinline__ void store_appended_piece(const StepParams& p, int row, int kvh, int lane, U32x4 x) {
  constexpr int LPR = ROWB / 16;
  GlobalU32x4* dst_k = global_uniform(p.k_pool);
  GlobalU32x4* dst_v = global_uniform(p.v_pool);
  const int slot = const_load(p.slots + row);
  if (lane < 2 * LPR && slot >= 0 && (int64_t)slot < (int64_t)p.num_blocks * 16) {
    const bool is_v = lane >= LPR;
    const int piece = lane - (is_v ? LPR : 0);
    (is_v ? dst_v : dst_k)[(((size_t)(slot >> 4) * p.num_kv_heads + kvh) * 16 + (slot & 15)) * LPR + piece] = x;
  }
}

// One workgroup of the decode kernel: query heads hx*GB .. hx*GB+GB-1 of
// sequence `seq`, partition `part` (the kernel's block indices; the step
// kernel of mixed steps runs the same workgroups among its own).
template <int KV, int QT, int D, int GB, bool FUSED = false>
__device__ __forceinline__ void decode_valu_wg(const StepParams& p, int hx, int seq, int part) {
  using T = Lay<KV, D>;
  static_assert(T::LPR >= 1 && T::LPR <= 16 && T::NL >= 1, "unsupported shape");
  static_assert(!T::DOT2 || KV == QT, "16-bit KV is read with q of the same type");

  const int lane = threadIdx.x & 63;
  // wave-uniform by construction; readfirstlane lets the compiler keep what derives
  // from it (block indices, buffer resources) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = p.num_q_heads / p.num_kv_heads;
  const int h0 = hx * GB;                        // first query head of this workgroup
  const int kvh = h0 / group;

  int row = seq;
  if (p.q_start != nullptr) {
    if (p.q_lens[seq] != 1) return;              // prefill chunks go to the chunk kernel
    row = p.q_start[seq];
    if (row < 0 || row >= p.total_q) return;
  }
  // Append taken into the decode step (16-bit KV): no workgroup of this launch
  // reads the new rows' slots from the pool; the partition holding position
  // L-1 attends to the row from k_new / v_new after the pool's blocks, in the
  // wave the round-robin would have given the next block.  The rows reach the
  // pool from the merge launch that follows when there is one
  // (append_in_merge), else from this launch: wave 0 of the partition-0
  // workgroup of the first head group of each kv head (the writer) stores the
  // row's new K and V into its slot, one 16-byte piece per lane (K on the
  // first LPR lanes, V on the next), whatever the row's length says.  Both
  // load their pieces before the walk and use them after it.
  static_assert(!FUSED || KV != kFP8, "the append goes into 16-bit decode launches only");
  const int L = p.ctx_lens[seq];
  const int tok0 = part_begin(part, p.part_tokens, p.part_head);
  const int tok_end = part_end(part, p.part_tokens, p.part_head);
  const bool bad = tok0 >= L || L > p.max_blocks * 16 || L + p.part_head > p.max_parts * p.part_tokens;
  bool writer = false, has_new = false;
  uint4 kn = make_uint4(0, 0, 0, 0), vn = make_uint4(0, 0, 0, 0);
  // each wave's copy of the new row (K, then V; lane l's piece at [l]), which
  // holds no registers across the walk
  __shared__ uint4 sm_new[FUSED ? kWaves : 1][2][64];
  if constexpr (FUSED) {
    writer = !p.append_in_merge && part == 0 && hx % (group / GB) == 0 && wave == 0;
    const int walked = max(0, min(L + 14, tok_end) / 16 - tok0 / 16);   // blocks of [tok0, L-1)
    has_new = !bad && wave == walked % kWaves && L - 1 >= tok0 && L - 1 < tok_end;
    // (LDS-destination buffer loads issued by every wave, moving bytes only
    // where needed: a branch around them would leave the compiler unsure, at
    // the block loop, which loads are still in flight)
    const size_t roff = ((size_t)row * p.num_kv_heads + kvh) * T::ROWB;
    const int new_bytes = __builtin_amdgcn_readfirstlane((writer || has_new) ? T::ROWB : 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(block_rsrc(p.k_new + roff, new_bytes),
                                             (__attribute__((address_space(3))) void*)sm_new[wave][0],
                                             16, (lane % T::LPR) * 16, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(block_rsrc(p.v_new + roff, new_bytes),
                                             (__attribute__((address_space(3))) void*)sm_new[wave][1],
                                             16, (lane % T::LPR) * 16, 0, 0, 0);
  }
  // this wave's pieces of the new row, once its loads have landed
  auto fetch_new = [&]() {
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    kn = sm_new[wave][0][lane];
    vn = sm_new[wave][1][lane];
  };
  // (the pieces passed by value: a lambda holding them by reference kept them
  // in private memory)
  auto store_new = [&](uint4 kv_k, uint4 kv_v) {
    const int slot = p.slots[row];
    if (lane < 2 * T::LPR && slot >= 0 && (int64_t)slot < (int64_t)p.num_blocks * 16) {
      const size_t dst = (((size_t)(slot >> 4) * p.num_kv_heads + kvh) * 16 + (slot & 15)) * T::ROWB +
                         (size_t)(lane % T::LPR) * 16;
      if (lane < T::LPR) *reinterpret_cast<uint4*>(const_cast<uint8_t*>(p.k_pool) + dst) = kv_k;
      else *reinterpret_cast<uint4*>(const_cast<uint8_t*>(p.v_pool) + dst) = kv_v;
    }
  };
  // rows whose length breaks the host scalars' promises are left unwritten
  if (bad) {
    if constexpr (FUSED) {
      if (writer) {
        fetch_new();
        store_new(kn, vn);
      }
    }
    return;
  }
  const int nparts = part_count(L, p.part_tokens, p.part_head);
  // tokens read from the pool (position L-1 comes from k_new / v_new when fused)
  const int Lw = FUSED ? L - 1 : L;
  const int blk_begin = tok0 >> 4;
  const int blk_end = min((Lw + 15) >> 4, tok_end >> 4);

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
    lim = i < end ? min(16, Lw - b * 16) : 0;
    if ((unsigned)phys >= (unsigned)p.num_blocks) { phys = 0; lim = 0; }
    const size_t boff = ((size_t)phys * p.num_kv_heads + kvh) * T::BLKB;
    // only the block's rows inside the context are read (none for a block with
    // no tokens; the count kept scalar: no waterfall loop)
    const int bytes = __builtin_amdgcn_readfirstlane(lim * T::ROWB);
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
  // the appended row, as a block of one token: every lane takes its piece of
  // the row, and only token row 0 counts
  if constexpr (FUSED) {
    if (has_new || writer) fetch_new();
    if (has_new) {
#pragma unroll
      for (int j = 0; j < T::NL; ++j) {
        kA[j] = kn;
        vA[j] = vn;
      }
      attend_block<KV, QT, D, GB>(kA, vA, 1.f, 1.f, 1, rg, qp, qf, p.scale_log2, m, l, acc);
    }
    if (writer) store_new(kn, vn);
  }

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

  // the GB partial rows of this workgroup lie max_parts rows apart, from the
  // first head's; fp8 KV keeps them as bfloat16, else float32
  constexpr int PB = KV == kFP8 ? 2 : 4;
  const size_t idx0 = ((size_t)row * p.num_q_heads + h0) * p.max_parts + part;
  const int64_t po_bytes = ((int64_t)(GB - 1) * p.max_parts + 1) * D * PB;
  const __amdgpu_buffer_rsrc_t po_res =
      block_rsrc(reinterpret_cast<const uint8_t*>(p.part_o) + idx0 * D * PB,
                 po_bytes < INT32_MAX ? (int)po_bytes : INT32_MAX);
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
      if constexpr (KV == kFP8) store_partial(po_res, (g * p.max_parts * D + d) * PB, to_out_bits<kBF16>(o));
      else store_partial(po_res, (g * p.max_parts * D + d) * PB, o);
      if (d == 0) {
        p.part_ml[idx * 2] = M;
        p.part_ml[idx * 2 + 1] = ls;
      }
    }
  }
}

}  // namespace pkv
