// MFMA attention tiles over paged KV for gfx950: the chunked-prefill tile and
// the grouped-query / fp8 decode.
//
// Page "Serving LLMs with vLLM: Continuous Batching and PagedAttention
// Explained", sections "Chunked Prefill" and "Prefill Versus Decode": a step
// mixes decoding sequences with a chunk of a long prompt whose rows attend
// causally to the sequence's paged history; section "Attention Over Scattered
// Blocks": the keys and values are fetched block by block through the table.
//
// A work item is (sequence, kv head, column tile, split-context partition).
// Its 16 columns are (query row, query head) pairs that read the same kv head:
// column c of the sequence is row c / G, head c % G (G = query heads per kv
// head), so a decode row with G = 8 fills 8 columns and a prefill chunk of an
// MHA model fills 16 rows.  Blocks are taken two at a time (32 tokens) and
// each product is a gfx950 16x16x32 MFMA:
//   S^T[token][col] = K[token][:] . Q[col][:]          (A = K, B = Q^T), per block
//   O^T[dim][col]  += V^T[dim][token] . P^T[token][col] (A = V^T, B = P^T), per pair
// The D-layout result of the first product (lane l: tokens 4*(l/16)..+3 of
// column l%16, for each block of the pair) is, with the pair's contraction
// index k = 8*(l/16) + i meaning token 4*(l/16) + i%4 of block i/4, exactly the
// B layout the second product needs, so the softmax weights never leave their
// lanes.  Head dims are permuted freely inside each contraction so that the
// operands are contiguous runs: for S^T, K chunk c of lane l holds the 16
// bytes at 64c + 16(l/16) of token row l%16 and the query operand holds the
// same dims (decode items load K as whole lines and regroup it into these
// chunks through LDS; prefill items read them from their LDS stages); for
// O^T from registers the output dim of (tile j, row m) is m * D/16 + j, so
// lane l reads D/16 consecutive dims of each of its tokens, and for O^T from
// LDS through transposing reads (16-bit prefill items) it is 16j + m.  fp8 K/V
// are converted to the query type in registers (exact: every e4m3 value is a
// bf16 and an f16), and
// the per-(block, head) scales are folded into the score (K) and the weight (V).
// Only the softmax weights are rounded on the way into the MFMA.  With 16-bit
// KV they enter as a 16-bit high part plus a 16-bit residual (two PV MFMAs per
// tile), so the products keep about 16 significant bits instead of 8; with fp8
// KV the values themselves carry 4 significant bits and the high part alone is
// well inside the error of the data.
#include "decode_valu.h"
#include "pkv_launch.h"

namespace pkv {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// D[16x16] += A[16x32] B[32x16]; lane l holds A[l%16][8*(l/16)..+7],
// B[8*(l/16)..+7][l%16] and D[4*(l/16)..+3][l%16]
template <int QT>
__device__ __forceinline__ f32x4 mfma32(uint4 a, uint4 b, f32x4 c) {
  if constexpr (QT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// D[16x16] += A[16x128] B[128x16] on fp8 E4M3 bytes: lane l holds 32 bytes of
// row l%16 of A and of column l%16 of B, with the same contraction indices in
// the same byte positions for A and B (so any consistent assignment of head
// dims to (lane group, byte) gives the dot product); D as in mfma32.  The
// E8M0 block scales are 127, i.e. 1.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma_fp8_128(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x4 c) {
  const i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8 b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// four floats -> four E4M3 bytes (round to nearest even), a in the lowest byte
__device__ __forceinline__ uint32_t f32x4_to_fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Query values as two fp8 operands whose sum is the value times 2^s: x (already
// scaled) -> hi = fp8(x), lo = fp8(x - hi).  A bfloat16 has 8 significant
// bits and hi keeps the top 4 (rounded), so x - hi is an exact float32 with at
// most 4 significant bits and lo = x - hi exactly, unless it falls below the
// fp8 normal range (|x - hi| < 2^-6; s puts the column's largest |x| in
// [128, 256), so only parts more than 2^13 below it lose bits).
__device__ __forceinline__ void split_fp8(const float (&x)[16], uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = f32x4_to_fp8x4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
    const auto b01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)h[i], false);
    const auto b23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)h[i], true);
    l[i] = f32x4_to_fp8x4(x[4 * i] - b01[0], x[4 * i + 1] - b01[1], x[4 * i + 2] - b23[0],
                          x[4 * i + 3] - b23[1]);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// two fp8 bytes (low or high half of w) -> two 16-bit values of type QT, packed
template <int QT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_16(uint32_t w) {
  if constexpr (QT == kBF16)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI));
}

// two floats -> two 16-bit values of type QT (round to nearest even), packed
template <int QT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (QT == kBF16) return f32x2_to_bf16x2(a, b);
  else return (uint32_t)to_out_bits<QT>(a) | ((uint32_t)to_out_bits<QT>(b) << 16);
}

template <int QT>
__device__ __forceinline__ float from_bits(uint16_t u) {
  if constexpr (QT == kBF16) return __uint_as_float((uint32_t)u << 16);
  else return (float)__builtin_bit_cast(_Float16, u);
}

// Softmax weights as the MFMA's 16-bit B operand, split hi + lo so that the
// product keeps ~16 significant bits: hi = round(w), lo = round(w - hi).
template <int QT>
__device__ __forceinline__ void split_weights(const float (&w)[8], uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack2<QT>(w[2 * i], w[2 * i + 1]);
    const float h0 = from_bits<QT>((uint16_t)h[i]);
    const float h1 = from_bits<QT>((uint16_t)(h[i] >> 16));
    l[i] = pack2<QT>(w[2 * i] - h0, w[2 * i + 1] - h1);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// select 16-bit halves: lo(x), lo(y) or hi(x), hi(y)
template <bool HI>
__device__ __forceinline__ uint32_t pick16(uint32_t x, uint32_t y) {
  return HI ? __builtin_amdgcn_perm(y, x, 0x07060302u) : __builtin_amdgcn_perm(y, x, 0x05040100u);
}

template <int KV, int D>
struct TileLay {
  static constexpr int ELT = (KV == kFP8) ? 1 : 2;
  static constexpr int ROWB = D * ELT;          // bytes of a token row of one head
  static constexpr int BLKB = 16 * ROWB;        // bytes of one (block, head)
  static constexpr int KSTEPS = D / 32;         // 16x16x32 MFMA steps of the score product
  // fp8 K at head_dim 128 with bf16 queries: scores on the fp8 16x16x128 MFMA
  // straight from the stored bytes (the query split exactly into two fp8
  // parts), no K conversions.  An f16 query has 11 significant bits, more
  // than two E4M3 parts hold, so f16 queries keep the conversion path.
  template <int QT>
  static constexpr bool f8mma() { return KV == kFP8 && D == 128 && QT == kBF16; }
  static constexpr int KB = D / 4 * ELT;        // K bytes per lane per block (D/4 dims)
  static constexpr int KLD = KB / 16;           // 16-byte chunks of K per lane
  // K chunk c of lane group gq holds bytes c*64 + gq*16 of its token row;
  // score step st contracts over the 8 dims starting at k_dim(st, gq), which
  // the query operand of that step holds too
  static __host__ __device__ constexpr int k_dim(int st, int gq) {
    return ELT == 2 ? st * 32 + gq * 8 : (st / 2) * 64 + gq * 16 + (st % 2) * 8;
  }
  static constexpr int CPR = ROWB / 16;         // 16-byte chunks per token row
  static constexpr int VB = D / 16 * ELT;       // V bytes per lane per token (D/16 dims)
  static constexpr int DT = D / 16;             // output dim tiles
  // blocks kept in the register ring (pairs of blocks are consumed together):
  // fp8 blocks are half as big, so one more pair is kept in flight
  static constexpr int NBUF = (KV == kFP8) ? 4 : 2;
  static_assert(KB % 16 == 0, "K slice must be whole 16-byte loads");
  static_assert(NBUF % 2 == 0, "blocks are consumed in pairs");
};

typedef uint32_t u32x2_buf __attribute__((ext_vector_type(2)));
// 32-bit word w of a token's V slice as loaded (VB bytes per lane)
template <int VB, typename T>
__device__ __forceinline__ uint32_t vword(const T& v, int w) {
  if constexpr (VB == 16) return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
  else if constexpr (VB == 8) return w == 0 ? v.x : v.y;
  else return v;
}
template <int VB> struct VVec;
template <> struct VVec<16> {
  typedef uint4 T;
  template <bool NT = false>
  static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int off) { return load_block16<NT>(r, off); }
  static __device__ __forceinline__ T lds(const uint4* base, int off) { return base[off / 16]; }
};
template <> struct VVec<8> {
  typedef uint2 T;
  template <bool NT = false>
  static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x2_buf v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, NT ? 2 : 0);
    return make_uint2(v.x, v.y);
  }
  static __device__ __forceinline__ T lds(const uint4* base, int off) {
    return reinterpret_cast<const uint2*>(base)[off / 8];
  }
};
template <> struct VVec<4> {
  typedef uint32_t T;
  template <bool NT = false>
  static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, NT ? 2 : 0);
  }
  static __device__ __forceinline__ T lds(const uint4* base, int off) {
    return reinterpret_cast<const uint32_t*>(base)[off / 4];
  }
};

// Stages of the LDS pipeline of prefill items.
constexpr int kStages = 4;

// LDS staging of prefill items: a stage is one pair of blocks, laid out as
// K0, K1, V0, V1 (each the block's (block, head) slice, BLKB bytes); two
// stages alternate.  K rows are stored with their 16-byte chunks permuted
// (chunk c of row r at c ^ key(r)) so that the 16 lanes reading one chunk
// index of 16 different rows hit 16 different bank groups; V is read along
// rows and kept as is.
template <int KV, int D>
struct StageLay {
  using L = TileLay<KV, D>;
  static constexpr int CHB = L::BLKB / 16;            // 16-byte chunks per block
  static constexpr int CHUNKS = 4 * CHB;              // per stage
  static constexpr int LOADS = CHUNKS / (kTileWaves * 64);   // 16-byte loads per thread
  static constexpr int CPR = L::ROWB / 16;            // chunks per token row
  static_assert(CHB % 64 == 0, "each wave's chunks of a stage lie in one block");
  static_assert(LOADS >= 1 && CHUNKS % (kTileWaves * 64) == 0, "whole loads per thread");
  static __device__ __forceinline__ int k_chunk(int row, int c) {
    return row * CPR + (c ^ ((row * CPR / 16) & (CPR - 1)));
  }
  // 16-bit V rows are read by transposing LDS reads, 32 bytes of each of 16
  // rows per 16-dim slice: chunk c of row r sits at c ^ (2r mod CPR), which
  // puts eight rows' chunk pairs in distinct bank groups
  static __device__ __forceinline__ int v_chunk(int row, int c) {
    return row * CPR + (c ^ ((2 * row) & (CPR - 1)));
  }
  // s_waitcnt immediate: at most n vector memory operations outstanding, no
  // LDS/scalar operation outstanding (gfx9 fields: vmcnt [3:0] and [15:14],
  // expcnt [6:4] left at its maximum, lgkmcnt [11:8] = 0)
  static constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
  static_assert((kStages - 2) * LOADS < 64, "outstanding copies fit the counter");
  // LDS of one stage; stage 0 also holds the decode items' merge buffer
  static constexpr int STAGE0 = CHUNKS > 2 * 16 * D / 4 ? CHUNKS : 2 * 16 * D / 4;
};

template <int KV, int D>
struct BlockRegs {
  using L = TileLay<KV, D>;
  uint4 k[L::KLD];
  typename VVec<L::VB>::T v[4];
  float ksc, vsc;
  int limit;     // tokens of the block that exist (0: nothing to score)
  int base;      // absolute position of the block's first token
};

struct TileItem {
  int seq, kvh, col0, ncols, part, part_tokens, part_head, L, Q, row0, max_parts;
};

// One work item for the whole workgroup.  SPLIT (decode rows): the item is
// one 16-column tile and the kTileWaves waves share the partition's blocks
// (wave w takes blocks w, w + kTileWaves, ...), merged through LDS at the end.
// !SPLIT (prefill chunks): the item is kTileWaves x TPW tiles of 16 columns,
// wave w owns tiles w*TPW .. w*TPW+TPW-1 and attends every block up to its
// last column's causal limit; the workgroup stages the blocks in LDS once for
// all four waves (st0..st3) and each wave writes its own columns.  With two
// tiles per wave a block's operand reads and fp8 conversions serve twice the
// matrix work.
// kst (decode items): this wave's LDS area of two blocks' K slices, through
// which K is regrouped from whole-line loads into the MFMA operand layout.
template <int KV, int QT, int D, bool SPLIT>
__device__ __forceinline__ void tile_item(const StepParams& p, const TileItem& it, int group,
                                          float* sm_o, float* sm_m, float* sm_l, uint4* st0 = nullptr,
                                          uint4* st1 = nullptr, uint4* st2 = nullptr,
                                          uint4* st3 = nullptr, uint4* kst = nullptr) {
  using L = TileLay<KV, D>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // scalar, provably
  const int n = lane & 15;          // column of this lane (token row of K it loads)
  const int gq = lane >> 4;         // lane group: tokens 4*gq..4*gq+3 / dims slice gq
  constexpr int TPW = tile_tiles_per_wave(KV, SPLIT);
  const int wcol0 = SPLIT ? it.col0 : it.col0 + 16 * TPW * wave;   // this wave's first column
  // (a wave of a prefill item with no columns still helps stage the blocks)
  int row[TPW], head[TPW], pos[TPW];
  bool col_ok[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int col = wcol0 + 16 * t + n;
    col_ok[t] = col < it.ncols;
    const int rloc = col_ok[t] ? col / group : 0;
    head[t] = it.kvh * group + (col_ok[t] ? col % group : 0);
    row[t] = it.row0 + rloc;
    pos[t] = it.L - it.Q + rloc;                          // last key this column sees
  }
  const int min_pos = it.L - it.Q + wcol0 / group;        // positions rise with the column
  const int last_col = min(wcol0 + 16 * TPW - 1, it.ncols - 1);
  const int max_pos = it.L - it.Q + last_col / group;
  const int tok0 = part_begin(it.part, it.part_tokens, it.part_head);
  const int tok1 = min(part_end(it.part, it.part_tokens, it.part_head), max_pos + 1);
  const int blk_begin = tok0 >> 4;
  const int blk_end = (tok1 + 15) >> 4;

  // Q^T operand of score step st: the 8 dims of this column's query that the
  // K operand of the same step holds (zero for unused columns)
  uint4 qb[TPW][L::KSTEPS];
  // fp8 scores (f8mma): the fp8 operands (hi, lo) of q * 2^s[t] over the dims the lane's K
  // chunks hold (16gq .. 16gq+15 and 64+16gq .. +15), and qs[t] = 2^-s[t],
  // which scales the scores back; s[t] puts the column's largest |q| in
  // [128, 256), inside the fp8 range.  qs is 1 on the other paths.
  uint4 qh[TPW][2], ql[TPW][2];
  float qs[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(p.q) + ((size_t)row[t] * p.num_q_heads + head[t]) * D;
    qs[t] = 1.f;
    if constexpr (L::template f8mma<QT>()) {
      float x[2][16];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          const uint4 raw = col_ok[t] ? *reinterpret_cast<const uint4*>(qrow + 64 * c + 16 * gq + 8 * h8)
                                      : make_uint4(0, 0, 0, 0);
          float f[8];
          if constexpr (QT == kBF16) unpack16<kBF16>(raw, f);
          else unpack16<kF16>(raw, f);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[c][8 * h8 + e] = f[e];
        }
      float amax = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[c][e]));
      amax = max_xor32(max_xor16(amax));            // the column's 4 lane groups
      int ex;
      (void)frexpf(amax, &ex);                      // amax = f * 2^ex, f in [0.5, 1)
      // (at most 2^100: a column whose largest |q| is below 2^-92 -- subnormal
      // bf16 included -- scores ~0 either way, and 2^(8 - ex) would overflow)
      const int sh = min(8 - ex, 100);
      const float up = ldexpf(1.f, sh);
      qs[t] = ldexpf(1.f, -sh);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[c][e] *= up;   // exact: a power of two
        split_fp8(x[c], qh[t][c], ql[t][c]);
      }
    } else {
#pragma unroll
      for (int st = 0; st < L::KSTEPS; ++st)
        qb[t][st] = col_ok[t] ? *reinterpret_cast<const uint4*>(qrow + L::k_dim(st, gq)) : make_uint4(0, 0, 0, 0);
    }
  }

  // this wave's blocks: blk_begin + first + stride * i, i < cnt
  constexpr int stride = SPLIT ? kTileWaves : 1;
  const int first = SPLIT ? wave : 0;
  const int32_t* trow = p.tables + (size_t)it.seq * p.max_blocks;
  const int nb = blk_end - blk_begin;
  const int cnt = nb > first ? (nb - first + stride - 1) / stride : 0;   // <= 256 (partition <= 4096)
  // prefill items: the blocks the workgroup stages, up to its last column's limit
  const int item_max_pos = it.L - it.Q + (it.ncols - 1) / group;
  const int cnt_item =
      max(0, ((min(part_end(it.part, it.part_tokens, it.part_head), item_max_pos + 1) + 15) >> 4) - blk_begin);
  const int tbl_cnt = SPLIT ? cnt : cnt_item;
  // Table entries (and fp8 scales) of the wave's blocks, read per block with
  // readlane.  Loading them up front keeps scalar loads out of the block loop:
  // a scalar load per block would be waited for together with every
  // prefetched block's (they complete out of order).  Decode items: lane l
  // holds block l.  Prefill items: lane l holds blocks 4l .. 4l+3, one per
  // word, so that the pairs of an unrolled round of the stage loop find their
  // entries in words known at compile time, and an entry is already the
  // (block, head) slice index, or -1 for an invalid block.
  constexpr int TW = SPLIT ? 1 : 4;
  int my_tbl[TW];
  float my_ks[TW], my_vs[TW];
#pragma unroll
  for (int w = 0; w < TW; ++w) {
    const int i = SPLIT ? lane + 64 * w : 4 * lane + w;
    my_tbl[w] = i < tbl_cnt ? trow[blk_begin + first + stride * i] : -1;
    my_ks[w] = 1.f;
    my_vs[w] = 1.f;
    const bool valid = (unsigned)my_tbl[w] < (unsigned)p.num_blocks;
    if constexpr (KV == kFP8) {
      if (valid) {
        my_ks[w] = p.k_scale[(size_t)my_tbl[w] * p.num_kv_heads + it.kvh];
        my_vs[w] = p.v_scale[(size_t)my_tbl[w] * p.num_kv_heads + it.kvh];
      }
    }
    if constexpr (!SPLIT) my_tbl[w] = valid ? my_tbl[w] * p.num_kv_heads + it.kvh : -1;
  }
  // Every word is read with readlane and the choice among them is made on the
  // scalar results: a select over the lane-held array itself was turned into
  // an indexed load from scratch memory, which then stalled each block's loads.
  auto lane_word = [&](const int (&a)[TW], int i) -> int {
    int v = __builtin_amdgcn_readlane(a[0], i & 63);
#pragma unroll
    for (int w = 1; w < TW; ++w) {
      const int x = __builtin_amdgcn_readlane(a[w], i & 63);
      v = (i >> 6) == w ? x : v;
    }
    return v;
  };
  auto lane_float = [&](const float (&a)[TW], int i) -> float {
    int v = __builtin_amdgcn_readlane(__float_as_int(a[0]), i & 63);
#pragma unroll
    for (int w = 1; w < TW; ++w) {
      const int x = __builtin_amdgcn_readlane(__float_as_int(a[w]), i & 63);
      v = (i >> 6) == w ? x : v;
    }
    return __int_as_float(v);
  };

  float m[TPW], lsum[TPW];
  f32x4 o[TPW][L::DT];
  // 16-bit prefill items: the running column sums come from one more MFMA
  // pair per tile with an all-ones A operand (D[m][n] = sum over k of the
  // weights, the same hi + lo weights the PV product uses), which moves eight
  // vector additions per tile and pair onto the matrix unit; each output row
  // then holds the sum, so no cross-lane reduction is needed at the end
  constexpr bool ONES_SUM = !SPLIT && KV != kFP8;
  f32x4 osum[TPW];
  const uint4 ones = QT == kBF16 ? make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u)
                                 : make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    m[t] = kMaxSeed;
    lsum[t] = 0.f;
    osum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < L::DT; ++j) o[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Every call issues the same loads with no branch around them: past the
  // wave's last block the index is clamped and the block counts no tokens (its
  // loads move no bytes), so the compiler can wait for exactly the block it
  // consumes instead of draining all outstanding loads at a control-flow join.
  // NT: nontemporal loads (blocks no other sequence of the step reads)
  auto issue = [&](auto nt_tag, int i, BlockRegs<KV, D>& r) {
    constexpr bool NT = decltype(nt_tag)::value;
    const int ic = min(i, cnt - 1);
    const int b = blk_begin + first + stride * ic;
    r.base = b * 16;
    r.ksc = 1.f;
    r.vsc = 1.f;
    int phys = lane_word(my_tbl, ic);
    r.limit = i < cnt ? min(16, it.L - b * 16) : 0;
    if ((unsigned)phys >= (unsigned)p.num_blocks) { phys = 0; r.limit = 0; }
    const size_t boff = ((size_t)phys * p.num_kv_heads + it.kvh) * L::BLKB;
    // only the block's existing token rows are in range: the rest (look-ahead
    // blocks entirely) read as zeros with no memory access, so no V slot past
    // the end needs a select (the count kept scalar: no waterfall loop)
    const int bytes = __builtin_amdgcn_readfirstlane(r.limit * L::ROWB);
    const __amdgpu_buffer_rsrc_t kres = block_rsrc(p.k_pool + boff, bytes);
    const __amdgpu_buffer_rsrc_t vres = block_rsrc(p.v_pool + boff, bytes);
    // K as whole lines: load c brings 16 bytes at c*1024 + 16*lane, so one
    // instruction reads 1 KiB of contiguous rows (regroup_k puts them in the
    // operand layout).  Loads of 64 bytes from each of 16 rows -- the operand
    // layout read straight from memory -- ran ~10% slower on their own.
#pragma unroll
    for (int c = 0; c < L::KLD; ++c) r.k[c] = load_block16<NT>(kres, c * 1024 + lane * 16);
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) r.v[i4] = VVec<L::VB>::template load<NT>(vres, (gq * 4 + i4) * L::ROWB + n * L::VB);
    if constexpr (KV == kFP8) {
      r.ksc = lane_float(my_ks, ic);
      r.vsc = lane_float(my_vs, ic);
    }
  };

  // Decode items: K of a block from its whole-line loads into the operand
  // layout (K chunk c of lane (n, gq) = bytes 64c + 16gq of token row n),
  // through the wave's own LDS area (no other wave touches it, and a wave's
  // LDS operations complete in order, so no barrier or wait is needed between
  // the writes and the reads).  Chunk j of row r is stored at j ^ (r mod CPR)
  // of its row: 8 consecutive lanes then write, and read, 8 distinct 16-byte
  // bank groups.  The wavefront-scope fences keep the compiler from moving
  // these accesses across one another (the reads take other lanes' writes,
  // and the next block's writes must follow this block's reads).
  auto regroup_k = [&](BlockRegs<KV, D>& r, uint4* area) {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
#pragma unroll
    for (int c = 0; c < L::KLD; ++c) {
      const int q = c * 64 + lane;                  // chunk index in the block
      const int row = q / L::CPR, j = q % L::CPR;
      area[row * L::CPR + (j ^ (row & (L::CPR - 1)))] = r.k[c];
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
#pragma unroll
    for (int c = 0; c < L::KLD; ++c) {
      const int j = 4 * c + gq;
      r.k[c] = area[n * L::CPR + (j ^ (n & (L::CPR - 1)))];
    }
  };

  // S^T for one block: 4 scores (tokens 4*gq..+3) of this lane's column in
  // every tile of the wave, each K operand built once
  auto scores = [&](const BlockRegs<KV, D>& r, f32x4 (&s)[TPW]) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (L::template f8mma<QT>()) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        s[t] = mfma_fp8_128(r.k[0], r.k[1], qh[t][0], qh[t][1], s[t]);
        s[t] = mfma_fp8_128(r.k[0], r.k[1], ql[t][0], ql[t][1], s[t]);
      }
      return;
    }
#pragma unroll
    for (int st = 0; st < L::KSTEPS; ++st) {
      uint4 a;
      if constexpr (KV == kFP8) {
        // 8 fp8 dims -> 8 16-bit values: half of a 16-byte load
        const uint4 raw = r.k[st / 2];
        const uint32_t w0 = (st & 1) ? raw.z : raw.x;
        const uint32_t w1 = (st & 1) ? raw.w : raw.y;
        a = make_uint4(fp8x2_to_16<QT, false>(w0), fp8x2_to_16<QT, true>(w0),
                       fp8x2_to_16<QT, false>(w1), fp8x2_to_16<QT, true>(w1));
      } else {
        a = r.k[st];
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) s[t] = mfma32<QT>(a, qb[t][st], s[t]);
    }
  };

  // the 16-bit V values of this lane's 4 tokens of a block (slots past the
  // block's end were read as zeros, so their weight 0 multiplies 0, never NaN)
  auto vvals = [&](const BlockRegs<KV, D>& r, uint32_t (&vw)[4][L::DT / 2]) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      if constexpr (KV == kFP8) {
        uint32_t raw[L::VB / 4];
        if constexpr (L::VB == 8) { raw[0] = r.v[i4].x; raw[1] = r.v[i4].y; }
        else { raw[0] = r.v[i4]; }
#pragma unroll
        for (int e = 0; e < L::VB / 4; ++e) {
          vw[i4][2 * e] = fp8x2_to_16<QT, false>(raw[e]);
          vw[i4][2 * e + 1] = fp8x2_to_16<QT, true>(raw[e]);
        }
      } else if constexpr (L::VB == 16) {
        vw[i4][0] = r.v[i4].x;
        vw[i4][1] = r.v[i4].y;
        vw[i4][2] = r.v[i4].z;
        vw[i4][3] = r.v[i4].w;
      } else {
        vw[i4][0] = r.v[i4].x;
        vw[i4][1] = r.v[i4].y;
      }
    }
  };

  // V^T operand of each 16-dim slice j from the V registers of a pair: the
  // 16-bit pairs (token t, token t+1) of dim 8n+j (n = lane's row of the
  // tile) for tokens 4gq..4gq+3 of r0 and of r1
  auto v_operand = [&](const BlockRegs<KV, D>& r0, const BlockRegs<KV, D>& r1, uint4 (&va)[L::DT]) {
    if constexpr (KV == kFP8) {
      // one byte permute gathers tokens t, t+1 at dims j, j+1; its two
      // conversions are then the operand words of slices j and j+1
#pragma unroll
      for (int j = 0; j < L::DT; j += 2) {
        const uint32_t b = j % 4;
        const uint32_t sel = b | ((4 + b) << 8) | ((b + 1) << 16) | ((5 + b) << 24);
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const BlockRegs<KV, D>& r = q < 2 ? r0 : r1;
          const int tk = (q & 1) * 2;
          const uint32_t x = vword<L::VB>(r.v[tk], j / 4);
          const uint32_t y = vword<L::VB>(r.v[tk + 1], j / 4);
          const uint32_t w = __builtin_amdgcn_perm(y, x, sel);
          lo[q] = fp8x2_to_16<QT, false>(w);
          hi[q] = fp8x2_to_16<QT, true>(w);
        }
        va[j] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        va[j + 1] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      }
    } else {
      uint32_t v0[4][L::DT / 2], v1[4][L::DT / 2];
      vvals(r0, v0);
      vvals(r1, v1);
#pragma unroll
      for (int j = 0; j < L::DT; ++j) {
        if (j & 1) {
          va[j].x = pick16<true>(v0[0][j / 2], v0[1][j / 2]);
          va[j].y = pick16<true>(v0[2][j / 2], v0[3][j / 2]);
          va[j].z = pick16<true>(v1[0][j / 2], v1[1][j / 2]);
          va[j].w = pick16<true>(v1[2][j / 2], v1[3][j / 2]);
        } else {
          va[j].x = pick16<false>(v0[0][j / 2], v0[1][j / 2]);
          va[j].y = pick16<false>(v0[2][j / 2], v0[3][j / 2]);
          va[j].z = pick16<false>(v1[0][j / 2], v1[1][j / 2]);
          va[j].w = pick16<false>(v1[2][j / 2], v1[3][j / 2]);
        }
      }
    }
  };

  // online softmax and PV over a pair of blocks (32 tokens).  DENSE: both
  // blocks are whole and every column of the wave sees all 32 tokens, so no
  // score is masked and the scale folds into the exponent's argument (for a
  // positive factor the maximum of the products is the product of the maximum).
  // build_va(va) fills the V^T operand of the pair.
  // Order: every tile's maximum and rescale factor first, then the one
  // (rarely taken) rescale branch, then per tile the weights and their PV
  // products -- straight-line code in which one tile's exponentials can be
  // issued between the other tile's matrix products.
  auto attend_pair = [&](auto dense_tag, const BlockRegs<KV, D>& r0, const BlockRegs<KV, D>& r1,
                         auto&& build_va) {
    constexpr bool DENSE = decltype(dense_tag)::value;
    f32x4 s0[TPW], s1[TPW];
    scores(r0, s0);
    scores(r1, s1);
    float mn[TPW], alpha[TPW];
    bool ok[TPW][8];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const float c0 = p.scale_log2 * qs[t] * r0.ksc, c1 = p.scale_log2 * qs[t] * r1.ksc;
      float mx;
      if constexpr (DENSE) {
        float mx0 = s0[t][0], mx1 = s1[t][0];
#pragma unroll
        for (int i = 1; i < 4; ++i) {
          mx0 = fmaxf(mx0, s0[t][i]);
          mx1 = fmaxf(mx1, s1[t][i]);
        }
        mx = max_xor32(max_xor16(fmaxf(mx0 * c0, mx1 * c1)));
      } else {
        mx = -__builtin_inff();
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int tk = gq * 4 + i4;
          ok[t][i4] = col_ok[t] && tk < r0.limit && r0.base + tk <= pos[t];
          ok[t][4 + i4] = col_ok[t] && tk < r1.limit && r1.base + tk <= pos[t];
          mx = fmaxf(mx, ok[t][i4] ? s0[t][i4] * c0 : -__builtin_inff());
          mx = fmaxf(mx, ok[t][4 + i4] ? s1[t][i4] * c1 : -__builtin_inff());
        }
        mx = max_xor32(max_xor16(mx));
      }
      mn[t] = mx > m[t] + kLazyRescale ? mx : m[t];   // lazy reference maximum
      alpha[t] = __builtin_amdgcn_exp2f(m[t] - mn[t]);
    }
    bool moved = false;
#pragma unroll
    for (int t = 0; t < TPW; ++t) moved = moved || alpha[t] != 1.f;
    if (__any(moved)) {     // the reference rarely moves after the first blocks
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
#pragma unroll
        for (int j = 0; j < L::DT; ++j) o[t][j] *= alpha[t];
        if constexpr (ONES_SUM) osum[t] *= alpha[t];
      }
    }

    uint4 va[L::DT];
    build_va(va);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const float c0 = p.scale_log2 * qs[t] * r0.ksc, c1 = p.scale_log2 * qs[t] * r1.ksc;
      float pw[8];
      if constexpr (DENSE) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pw[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[t][i], c0, -mn[t]));
          pw[4 + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[t][i], c1, -mn[t]));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pw[i] = ok[t][i] ? __builtin_amdgcn_exp2f(s0[t][i] * c0 - mn[t]) : 0.f;
          pw[4 + i] = ok[t][4 + i] ? __builtin_amdgcn_exp2f(s1[t][i] * c1 - mn[t]) : 0.f;
        }
      }
      if constexpr (!ONES_SUM) {       // (else the column sums come out of the MFMA below)
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ps += pw[i];
        lsum[t] = lsum[t] * alpha[t] + ps;
      }
      m[t] = mn[t];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pw[i] *= r0.vsc;
        pw[4 + i] *= r1.vsc;
      }
      uint4 pb_hi, pb_lo;
      split_weights<QT>(pw, pb_hi, pb_lo);
      if constexpr (ONES_SUM) {
        osum[t] = mfma32<QT>(ones, pb_hi, osum[t]);
        osum[t] = mfma32<QT>(ones, pb_lo, osum[t]);
      }
#pragma unroll
      for (int j = 0; j < L::DT; ++j) {
        o[t][j] = mfma32<QT>(va[j], pb_hi, o[t][j]);
        if constexpr (KV != kFP8) o[t][j] = mfma32<QT>(va[j], pb_lo, o[t][j]);
      }
    }
  };

  // The wave's blocks rise in position, so the dense pairs (both blocks wholly
  // at or before min_pos) form a prefix of its block list.
  const int vis_blocks = (min_pos + 1) >> 4;   // blocks 0 .. vis_blocks-1 end at or before min_pos
  const int dense_blocks = min(cnt, max(0, vis_blocks - blk_begin - first + stride - 1) / stride);
  constexpr int NB = L::NBUF;
  constexpr int NP = NB / 2;
  if constexpr (SPLIT) {
  // Decode items: a register ring in which NB/2 - 1 pairs are loading while
  // the current pair is scored; pairs past the end (at most NB/2 - 1 per wave)
  // are scored fully masked.  The dense prefix runs in a loop of its own, cut
  // to a multiple of the ring's pairs so the loops use the same register slots.
  // Each block of a decode item is read by one wave only, so the blocks are
  // streamed past the caches (nontemporal loads), except the leading blocks
  // the caller marks as shared with other sequences of the step (a prefix
  // that other waves read too stays cached).  Pairs [0, shared_pairs) load
  // cached, the rest nontemporal (both ends cut to whole rounds of the ring).
  BlockRegs<KV, D> buf[NB];
  if (cnt > 0) {
    const int npairs = (cnt + 1) / 2;
    const int dense_pairs = dense_blocks / 2 / NP * NP;
    const int hint = p.shared_blocks != nullptr ? uniform_load(p.shared_blocks + it.seq) : 0;
    const int nsh = min(max(hint, blk_begin), blk_end);      // clamped before any arithmetic
    const int cnt_sh = min(cnt, max(0, nsh - blk_begin - first + stride - 1) / stride);
    const int shared_pairs = min((cnt_sh + 1) / 2 + NP - 1, dense_pairs) / NP * NP;
#pragma unroll
    for (int k = 0; k < NP - 1; ++k) {
      if (shared_pairs > 0) {
        issue(std::false_type{}, 2 * k, buf[2 * k]);
        issue(std::false_type{}, 2 * k + 1, buf[2 * k + 1]);
      } else {
        issue(std::true_type{}, 2 * k, buf[2 * k]);
        issue(std::true_type{}, 2 * k + 1, buf[2 * k + 1]);
      }
    }
    auto run = [&](auto dense_tag, auto nt_tag, int q_begin, int q_end) {
      for (int q2 = q_begin; q2 < q_end; q2 += NP) {
#pragma unroll
        for (int u = 0; u < NP; ++u) {
          const int nxt = q2 + u + NP - 1;
          const int slot = (u + NP - 1) % NP;
          issue(nt_tag, 2 * nxt, buf[2 * slot]);
          issue(nt_tag, 2 * nxt + 1, buf[2 * slot + 1]);
          regroup_k(buf[2 * u], kst);
          regroup_k(buf[2 * u + 1], kst + L::BLKB / 16);
          attend_pair(dense_tag, buf[2 * u], buf[2 * u + 1],
                      [&](uint4 (&va)[L::DT]) { v_operand(buf[2 * u], buf[2 * u + 1], va); });
        }
      }
    };
    run(std::true_type{}, std::false_type{}, 0, shared_pairs);
    run(std::true_type{}, std::true_type{}, shared_pairs, dense_pairs);
    run(std::false_type{}, std::true_type{}, dense_pairs, npairs);
  }
  } else {
    // Prefill item: the four waves read the same blocks, so the workgroup
    // stages each pair once in LDS and every wave builds its operands from
    // there.  Blocks go straight from memory into LDS (buffer loads with the
    // LDS destination: no registers held while they travel), kStages stages
    // deep: pair q+kStages-1 is requested while pair q is attended.  Each
    // stage is an LDS array of its own and the loop is unrolled over them, so
    // the compiler can tell which outstanding copies a read depends on.  One
    // barrier per pair: a wave first waits for its own copies of pair q (and
    // for its reads of the previous pair), so after the barrier the whole
    // pair is in place and the stage read before it is free for reuse.  All
    // waves step through the item's pairs (a wave stops attending past its
    // own last column).
    using SL = StageLay<KV, D>;
    constexpr int S = kStages;
    constexpr bool VTR = KV != kFP8;    // 16-bit V: transposing LDS reads
    const int np_item = (cnt_item + 1) / 2;
    const bool has_cols = wcol0 < it.ncols;
    const int np_w = has_cols ? (cnt + 1) / 2 : 0;
    const int dense_pairs = has_cols ? dense_blocks / 2 : 0;
    // tokens held by block i of the item
    auto tokens = [&](int i) { return i < cnt_item ? min(16, it.L - (blk_begin + i) * 16) : 0; };
    // block 2q+j: lane q/2 holds it in word 2(q%2)+j, and q%2 = u%2 for the
    // step u of a round (rounds start at multiples of S)
    auto entry = [&](const auto& a, int q, int j, int u) -> int {
      return __builtin_amdgcn_readlane(__builtin_bit_cast(int, a[2 * (u & 1) + j]), (q >> 1) & 63);
    };
    // Copy pair q into a stage.  Wave w moves chunk groups g = k*4 + w (64
    // chunks each, all within block g*64/CHB of the stage); lane l fills LDS
    // chunk g*64 + l, fetching the K chunk the row permutation puts there.
    // Rows past the block's tokens (all rows of a block past the item's end
    // or with an invalid table entry) are out of the buffer's range.
    auto copy_pair = [&](int q, int u, uint4* stage) {
      int ent[2], bytes[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        ent[j] = entry(my_tbl, q, j, u);
        bytes[j] = __builtin_amdgcn_readfirstlane(ent[j] >= 0 ? tokens(2 * q + j) * L::ROWB : 0);
      }
#pragma unroll
      for (int k = 0; k < SL::LOADS; ++k) {
        const int g = k * kTileWaves + wave;
        // g * 64 / CHB, written so that it is a constant when a block spans
        // all four waves' chunk groups (wave < 4)
        constexpr int CPB = SL::CHB / 64;
        const int bi = CPB == kTileWaves ? k : g / CPB;
        const int d = (g * 64) % SL::CHB + lane;
        const int row = d / SL::CPR, c = d % SL::CPR;
        const int goff = (bi < 2 ? SL::k_chunk(row, c) : (VTR ? SL::v_chunk(row, c) : d)) * 16;
        const int e = (bi & 1) ? ent[1] : ent[0];
        const size_t boff = (size_t)(uint32_t)max(e, 0) * L::BLKB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            block_rsrc((bi < 2 ? p.k_pool : p.v_pool) + boff, (bi & 1) ? bytes[1] : bytes[0]),
            (__attribute__((address_space(3))) void*)(stage + g * 64), 16, goff, 0, 0, 0);
      }
    };
    // block j of pair q from a stage, in the register layout the ring uses
    // (an invalid table entry is not masked here: a caller error gives wrong
    // numbers, never an access outside the pools)
    auto from_stage = [&](const uint4* stage, int q, int j, int u, BlockRegs<KV, D>& r) {
      const uint4* kb = stage + j * SL::CHB;
      const uint4* vb = stage + (2 + j) * SL::CHB;
#pragma unroll
      for (int c = 0; c < L::KLD; ++c) r.k[c] = kb[SL::k_chunk(n, c * 4 + gq)];
      if constexpr (!VTR) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) r.v[i4] = VVec<L::VB>::lds(vb, (gq * 4 + i4) * L::ROWB + n * L::VB);
      }
      r.base = (blk_begin + 2 * q + j) * 16;
      r.limit = tokens(2 * q + j);
      r.ksc = 1.f;
      r.vsc = 1.f;
      if constexpr (KV == kFP8) {
        r.ksc = __int_as_float(entry(my_ks, q, j, u));
        r.vsc = __int_as_float(entry(my_vs, q, j, u));
      }
    };
    // 16-bit V operand straight from the stage with transposing LDS reads:
    // within each 16-lane group, lane d of the result gets element d%4 of the
    // 8 bytes read by lanes 4k + d/4 (k = 0..3), so when lane (s, g) reads
    // dims 16j + 4(s%4) .. +3 of token row 4g + s/4, lane (d, g) receives
    // dim 16j + d of tokens 4g .. 4g+3: the A operand rows are the slice's 16
    // dims (output row m of slice j is dim 16j + m) and the tokens line up
    // with the weights' k slots, first block then second.
    auto v_operand_tr = [&](const uint4* stage, uint4 (&va)[L::DT]) {
      const int row = 4 * gq + (n >> 2);
#pragma unroll
      for (int j = 0; j < L::DT; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const uint4* vb = stage + (2 + b) * SL::CHB;
          const int c = 2 * j + ((n & 3) >> 1);
          const int byte = SL::v_chunk(row, c) * 16 + 8 * (n & 1);
          typedef short v4s __attribute__((ext_vector_type(4)));
          const v4s t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)((__attribute__((address_space(3))) char*)vb + byte));
          w[2 * b] = (uint32_t)(uint16_t)t[0] | ((uint32_t)(uint16_t)t[1] << 16);
          w[2 * b + 1] = (uint32_t)(uint16_t)t[2] | ((uint32_t)(uint16_t)t[3] << 16);
        }
        va[j] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    };
    uint4* const stage[4] = {st0, st1, st2, st3};
    if (cnt_item > 0) {
      // the previous item's reads of the stages and its copies are done
      __builtin_amdgcn_s_waitcnt(kWaitAll);
      __builtin_amdgcn_s_barrier();
      // Copies are issued without conditions (a pair past the item's end
      // moves no bytes and is never read), so every step leaves exactly S-1
      // pairs in flight and the compiler's count of them stays exact.
#pragma unroll
      for (int k = 0; k < S - 1; ++k) copy_pair(k, k, stage[k]);
      // pairs [0, dense_end): whole blocks every column sees (cut to whole
      // rounds of the stages); then the rest, masked, in whole rounds
      auto run = [&](auto dense_tag, int q_begin, int q_end) {
        for (int q0 = q_begin; q0 < q_end; q0 += S) {
#pragma unroll
          for (int u = 0; u < S; ++u) {
            const int q = q0 + u;
            // own copies of pair q landed (later pairs may still travel),
            // own reads of pair q-1 done; then the workgroup's barrier
            __builtin_amdgcn_s_waitcnt(SL::wait_vm((S - 2) * SL::LOADS));
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
            copy_pair(q + S - 1, u + S - 1, stage[(u + S - 1) % S]);
            if (q < np_w) {
              BlockRegs<KV, D> r0, r1;
              from_stage(stage[u], q, 0, u, r0);
              from_stage(stage[u], q, 1, u, r1);
              attend_pair(dense_tag, r0, r1, [&](uint4 (&va)[L::DT]) {
                if constexpr (VTR) v_operand_tr(stage[u], va);
                else v_operand(r0, r1, va);
              });
            }
          }
        }
      };
      const int dense_end = dense_pairs / S * S;
      run(std::true_type{}, 0, dense_end);
      run(std::false_type{}, dense_end, np_item);
    }
  }

  // the column's running sum is spread over the 4 lane groups
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if constexpr (ONES_SUM) lsum[t] = osum[t][0];   // every output row holds the column sum
    else lsum[t] = sum_xor32(sum_xor16(lsum[t]));
  }

  if constexpr (SPLIT) {
    // Merge the four waves' partials of the same 16 columns in two rounds
    // through 2 x 16 x D floats of LDS (waves 2, 3 -> 0, 1, then 1 -> 0), half
    // of what one round needs; the LDS then no longer caps the workgroups a
    // CU holds below what the registers allow.
    auto put = [&](int slot) {
#pragma unroll
      for (int j = 0; j < L::DT; ++j)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) sm_o[(slot * 16 + n) * D + (gq * 4 + i4) * L::DT + j] = o[0][j][i4];
      if (gq == 0) {
        sm_m[slot * 16 + n] = m[0];
        sm_l[slot * 16 + n] = lsum[0];
      }
    };
    auto take = [&](int slot) {
      const float m2 = sm_m[slot * 16 + n];
      const float M = fmaxf(m[0], m2);
      const float f1 = __builtin_amdgcn_exp2f(m[0] - M);
      const float f2 = __builtin_amdgcn_exp2f(m2 - M);
      lsum[0] = lsum[0] * f1 + sm_l[slot * 16 + n] * f2;
#pragma unroll
      for (int j = 0; j < L::DT; ++j)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          o[0][j][i4] = o[0][j][i4] * f1 + sm_o[(slot * 16 + n) * D + (gq * 4 + i4) * L::DT + j] * f2;
      m[0] = M;
    };
    if (wave >= 2) put(wave - 2);
    __syncthreads();
    if (wave < 2) take(wave);
    __syncthreads();
    if (wave == 1) put(0);
    __syncthreads();
    if (wave != 0) return;
    take(0);
  }

  // head dim of output row 4gq+i4 of slice j: 16j + row where V came through
  // transposing reads (16-bit prefill items), else 8*row + j
  auto out_dim = [&](int j, int i4) {
    if constexpr (!SPLIT && KV != kFP8) return 16 * j + gq * 4 + i4;
    else return (gq * 4 + i4) * L::DT + j;
  };
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    // this wave holds its columns' result over the partition: write it out
    if (!col_ok[t] || pos[t] < tok0) continue;     // no key of this partition is visible
    const size_t rh = (size_t)row[t] * p.num_q_heads + head[t];
    const int nparts = part_count(pos[t] + 1, it.part_tokens, it.part_head);
    if (nparts == 1 && !p.new_in_merge) {
      const float inv = 1.f / lsum[t];
      uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) + rh * D;
#pragma unroll
      for (int j = 0; j < L::DT; ++j)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) orow[out_dim(j, i4)] = to_out_bits<QT>(o[t][j][i4] * inv);
    } else {
      const size_t idx = rh * it.max_parts + it.part;
      if constexpr (KV == kFP8) {
        // bfloat16 partials: the DT dims of (gq, i4) are consecutive, so each
        // goes out as one DT * 2-byte store
        static_assert(L::DT == 4 || L::DT == 8, "one 8- or 16-byte store per (gq, i4)");
        uint16_t* po = reinterpret_cast<uint16_t*>(p.part_o) + idx * D;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          uint32_t w[L::DT / 2];
#pragma unroll
          for (int j = 0; j < L::DT; j += 2) w[j / 2] = f32x2_to_bf16x2(o[t][j][i4], o[t][j + 1][i4]);
          if constexpr (L::DT == 8)
            *reinterpret_cast<uint4*>(po + out_dim(0, i4)) = make_uint4(w[0], w[1], w[2], w[3]);
          else
            *reinterpret_cast<uint2*>(po + out_dim(0, i4)) = make_uint2(w[0], w[1]);
        }
      } else {
        float* po = p.part_o + idx * D;
#pragma unroll
        for (int j = 0; j < L::DT; ++j)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) po[out_dim(j, i4)] = o[t][j][i4];
      }
      if (gq == 0) {
        p.part_ml[idx * 2] = m[t];
        p.part_ml[idx * 2 + 1] = lsum[t];
      }
    }
  }
}

// Decode rows (and sequences with at most small_q query rows, e.g. the rows a
// speculative-decoding step verifies): one work item per (kv head x column
// tile, sequence, partition) coordinate; the sequence's query_len * G columns
// fill the tiles and the 4 waves share the partition's blocks.
template <int KV, int QT, int D>
__device__ __forceinline__ void decode_wg(const StepParams& p, int x, int seq, int part,
                                          float* sm_o, float* sm_m, float* sm_l, uint4* kst) {
  const int group = p.num_q_heads / p.num_kv_heads;
  const int tiles = (p.small_q * group + 15) / 16;
  TileItem it;
  it.seq = seq;
  it.kvh = x / tiles;
  it.col0 = (x % tiles) * 16;
  it.part = part;
  it.part_tokens = p.part_tokens;
  it.part_head = p.part_head;
  it.max_parts = p.max_parts;
  it.Q = 1;
  if (p.q_start != nullptr) {
    it.Q = uniform_load(p.q_lens + it.seq);
    if (it.Q < 1 || it.Q > p.small_q) return;      // longer prefill chunks are chunk items
    it.row0 = uniform_load(p.q_start + it.seq);
    if (it.row0 < 0 || it.row0 + it.Q > p.total_q) return;
  } else {
    it.row0 = it.seq;
  }
  it.ncols = it.Q * group;
  if (it.col0 >= it.ncols) return;
  it.L = uniform_load(p.ctx_lens + it.seq);
  if (it.Q > it.L || it.L > p.max_blocks * 16 || it.L + it.part_head > p.max_parts * it.part_tokens) return;
  // the merge launch adds key L-1 (this step's new row) from k_new / v_new
  if (p.new_in_merge) it.L -= 1;
  if (it.Q > it.L || part_begin(it.part, it.part_tokens, it.part_head) >= it.L) return;
  tile_item<KV, QT, D, true>(p, it, group, sm_o, sm_m, sm_l, nullptr, nullptr, nullptr, nullptr, kst);
}

// Prefill chunks (query_len > 1): the prologue lists (sequence, first column)
// entries of chunk_cols columns each; `nwg` workgroups starting at `wg` stride over
// entries x kv heads x partitions.
template <int KV, int QT, int D>
__device__ __forceinline__ void chunk_wgs(const StepParams& p, int wg, int nwg, float* sm_o,
                                          float* sm_m, float* sm_l, uint4* st0, uint4* st1,
                                          uint4* st2, uint4* st3) {
  const int group = p.num_q_heads / p.num_kv_heads;
  const int n_entries = min(uniform_load(p.chunk_count), p.chunk_capacity);
  const int per_entry = p.num_kv_heads * p.chunk_max_parts;
  const long long items = (long long)n_entries * per_entry;
  for (long long item = wg; item < items; item += nwg) {
    // entries are listed by rising column within each sequence, and a later
    // column attends more keys: taking them last to first hands out the
    // longest items first, so the launch does not end on a few long ones
    const int eo = (int)(item / per_entry);
    const int rem = (int)(item - (long long)eo * per_entry);
    const int e = n_entries - 1 - eo;
    TileItem it;
    it.seq = uniform_load(p.chunk_entries + 2 * e);
    it.col0 = uniform_load(p.chunk_entries + 2 * e + 1);
    it.kvh = rem / p.chunk_max_parts;
    it.part = rem - it.kvh * p.chunk_max_parts;
    it.part_tokens = p.chunk_part_tokens;
    it.part_head = 0;
    it.max_parts = p.max_parts;
    if ((unsigned)it.seq >= (unsigned)p.num_seqs) continue;
    it.Q = uniform_load(p.q_lens + it.seq);
    it.L = uniform_load(p.ctx_lens + it.seq);
    it.row0 = uniform_load(p.q_start + it.seq);
    it.ncols = it.Q * group;
    if (it.Q < 1 || it.Q > it.L || it.L > p.max_blocks * 16 || it.row0 < 0 ||
        it.row0 + it.Q > p.total_q || it.col0 >= it.ncols)
      continue;
    const int last_col = min(it.col0 + p.chunk_cols - 1, it.ncols - 1);
    const int max_pos = it.L - it.Q + last_col / group;
    if (it.part * it.part_tokens > max_pos || max_pos + 1 > p.max_parts * it.part_tokens) continue;
    tile_item<KV, QT, D, false>(p, it, group, sm_o, sm_m, sm_l, st0, st1, st2, st3);
  }
}

// Decode rows only: grid.x = kv head x column tile (fastest), then sequence;
// grid.y = partition, in the order set by dispatch_part.
template <int KV, int QT, int D>
__global__ __launch_bounds__(kTileWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void decode_mfma_kernel(StepParams p) {
  __shared__ float sm_o[2 * 16 * D];
  __shared__ float sm_m[2 * 16];
  __shared__ float sm_l[2 * 16];
  // each wave's K regrouping area: two blocks' K slices
  __shared__ uint4 sm_k[kTileWaves * 2 * TileLay<KV, D>::BLKB / 16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nx = p.num_kv_heads * ((p.small_q * (p.num_q_heads / p.num_kv_heads) + 15) / 16);
  const int seq = blockIdx.x / nx;
  decode_wg<KV, QT, D>(p, blockIdx.x - seq * nx, seq, dispatch_part(p), sm_o, sm_m, sm_l,
                       sm_k + wave * 2 * TileLay<KV, D>::BLKB / 16);
}

// A step with prefill chunks: one launch runs the chunk work items and the
// decode work items, interleaved in dispatch order (one chunk workgroup every
// `stride` ids) so that the chunks' MFMA work overlaps the decode rows' HBM
// traffic across the whole launch.  Decode ids decode as x fastest, then
// sequence, then partition.  VGB = 0: decode items are MFMA tiles (x = kv
// head x column tile); VGB = 1 or 2: single-row sequences run as the VALU
// decode kernel's workgroups of VGB query heads (x = head group), which hold
// their HBM rate at this kernel's two waves per SIMD.
template <int KV, int QT, int D, int VGB>
__global__ __launch_bounds__(kTileWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void step_mfma_kernel(StepParams p, int n_chunk_wgs,
                                                                   int stride, int dec_x, int dec_y) {
  // four stage arrays (a decode item's merge buffer lives in the first)
  __shared__ uint4 st0[StageLay<KV, D>::STAGE0];
  __shared__ uint4 st1[StageLay<KV, D>::CHUNKS];
  __shared__ uint4 st2[StageLay<KV, D>::CHUNKS];
  __shared__ uint4 st3[StageLay<KV, D>::CHUNKS];
  __shared__ float sm_m[2 * 16];
  __shared__ float sm_l[2 * 16];
  float* sm_o = reinterpret_cast<float*>(st0);
  const int b = blockIdx.x;
  const int k = b / stride;
  const int r = b - k * stride;
  int id;
  if (k < n_chunk_wgs) {
    if (r == 0) {
      chunk_wgs<KV, QT, D>(p, k, n_chunk_wgs, sm_o, sm_m, sm_l, st0, st1, st2, st3);
      return;
    }
    id = k * (stride - 1) + (r - 1);
  } else {
    id = n_chunk_wgs * (stride - 1) + (b - n_chunk_wgs * stride);
  }
  const int x = id % dec_x;
  const int y = (id / dec_x) % dec_y;
  const int z = id / (dec_x * dec_y);
  if constexpr (VGB > 0) decode_valu_wg<KV, QT, D, VGB>(p, x, y, z);
  else {
    // decode items regroup K in the prefill stages 1 and 2 (4 blocks each), two
    // blocks per wave; a workgroup runs either a prefill item or a decode item
    static_assert(StageLay<KV, D>::CHUNKS >= 4 * TileLay<KV, D>::BLKB / 16, "stage holds 4 blocks");
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    decode_wg<KV, QT, D>(p, x, y, z, sm_o, sm_m, sm_l,
                         (wave < 2 ? st1 : st2) + (wave & 1) * 2 * TileLay<KV, D>::BLKB / 16);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// vgb: 0, or the VALU decode workgroup's query heads (16-bit KV only)
template <int KV, int QT, int D>
static void launch_tile_kernel(bool step, int vgb, const StepParams& p, dim3 grid, int n_chunk,
                               int dx, int dy, hipStream_t stream) {
  const dim3 block(kTileWaves * 64);
  if (step) {
    const int stride = n_chunk > 0 ? (int)(grid.x / (uint32_t)n_chunk) : 1;
    if constexpr (KV != kFP8) {
      if (vgb == 1) {
        hipLaunchKernelGGL((step_mfma_kernel<KV, QT, D, 1>), grid, block, 0, stream, p, n_chunk,
                           stride, dx, dy);
        return;
      }
      if (vgb == 2) {
        hipLaunchKernelGGL((step_mfma_kernel<KV, QT, D, 2>), grid, block, 0, stream, p, n_chunk,
                           stride, dx, dy);
        return;
      }
    }
    hipLaunchKernelGGL((step_mfma_kernel<KV, QT, D, 0>), grid, block, 0, stream, p, n_chunk, stride,
                       dx, dy);
  } else
    hipLaunchKernelGGL((decode_mfma_kernel<KV, QT, D>), grid, block, 0, stream, p);
}

template <int KV, int QT>
static hipError_t launch_tile(bool step, int vgb, const StepParams& p, int head_dim, dim3 grid,
                              int n_chunk, int dx, int dy, hipStream_t stream) {
  (void)hipGetLastError();   // drop an error some earlier, unrelated call left behind
  if (head_dim == 128) launch_tile_kernel<KV, QT, 128>(step, vgb, p, grid, n_chunk, dx, dy, stream);
  else launch_tile_kernel<KV, QT, 64>(step, vgb, p, grid, n_chunk, dx, dy, stream);
  return hipGetLastError();
}

static hipError_t launch_tile_typed(bool step, int vgb, const StepParams& p, const StepPlan& plan,
                                    dim3 grid, int n_chunk, int dx, int dy, hipStream_t stream) {
  if (plan.q_dtype == kBF16) {
    if (plan.kv_dtype == kBF16) return launch_tile<kBF16, kBF16>(step, vgb, p, plan.head_dim, grid, n_chunk, dx, dy, stream);
    if (plan.kv_dtype == kFP8) return launch_tile<kFP8, kBF16>(step, vgb, p, plan.head_dim, grid, n_chunk, dx, dy, stream);
  } else if (plan.q_dtype == kF16) {
    if (plan.kv_dtype == kF16) return launch_tile<kF16, kF16>(step, vgb, p, plan.head_dim, grid, n_chunk, dx, dy, stream);
    if (plan.kv_dtype == kFP8) return launch_tile<kFP8, kF16>(step, vgb, p, plan.head_dim, grid, n_chunk, dx, dy, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(const StepParams& p, const StepPlan& plan, hipStream_t stream) {
  const int tiles = (p.small_q * plan.group + 15) / 16;
  const dim3 grid((uint32_t)(p.num_kv_heads * tiles * p.num_seqs), (uint32_t)p.max_parts);
  return launch_tile_typed(false, 0, p, plan, grid, 0, 0, 0, stream);
}

hipError_t launch_step_mfma(const StepParams& p, const StepPlan& plan, hipStream_t stream) {
  // decode rows as VALU decode workgroups (plan.decode_on_mfma false: 16-bit KV,
  // at most two query heads per kv head) or as MFMA tiles
  const int vgb = plan.decode_on_mfma ? 0 : plan.heads_per_wg;
  if (vgb != 0 && (plan.kv_dtype == kFP8 || vgb > 2)) return hipErrorInvalidValue;
  const int tiles = (p.small_q * plan.group + 15) / 16;
  const int dx = vgb ? p.num_q_heads / vgb : p.num_kv_heads * tiles;
  const int dy = p.num_seqs;
  const long long dec = (long long)dx * dy * p.max_parts;
  const long long total = dec + plan.chunk_grid;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  return launch_tile_typed(true, vgb, p, plan, dim3((uint32_t)total), plan.chunk_grid, dx, dy, stream);
}

}  // namespace pkv
