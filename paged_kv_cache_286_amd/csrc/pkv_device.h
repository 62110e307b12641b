// Device-side helpers shared by the gfx950 kernels of libpagedkv.
// Element conversions, wave64 reductions and the parameter block of one step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// element type codes (same values as pkv_dtype)
constexpr int kF16 = 0;
constexpr int kBF16 = 1;
constexpr int kFP8 = 2;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
// running-max seed: finite, far below any real score, so exp2(seed - seed) = 1 and
// exp2(seed - real) = 0 without ever forming inf - inf
constexpr float kMaxSeed = -1.0e30f;
// An online-softmax reference maximum may lag the true running maximum by up to
// this much (log2 units): weights are then at most 2^kLazyRescale, numerator and
// denominator share the reference, and the accumulators are rescaled only when
// a score passes the reference by more than this.
constexpr float kLazyRescale = 8.0f;

// violation codes of the checks build (same values as pkv_violation)
constexpr int kViolationNone = 0;
constexpr int kViolationBlockId = 1;
constexpr int kViolationContextLen = 2;
constexpr int kViolationQueryLen = 3;
constexpr int kViolationTotalRows = 4;

// ---------------------------------------------------------------------------
// parameters of one paged_attn_step, as the kernels see them
// ---------------------------------------------------------------------------
// The MFMA tile kernel: kTileWaves waves per workgroup; a prefill-chunk work
// item gives each wave tile_tiles_per_wave 16-column tiles (two; one for the
// decode items, which split their blocks over the waves instead), so an entry
// of the prologue's list covers chunk_entry_cols (row, head) columns.
constexpr int kTileWaves = 4;
constexpr int tile_tiles_per_wave(int, bool split) { return split ? 1 : 2; }
constexpr int chunk_entry_cols(int kv_dtype) { return 16 * kTileWaves * tile_tiles_per_wave(kv_dtype, false); }

struct StepParams {
  const void* q;             // [Tq][Hq][D]
  void* out;                 // [Tq][Hq][D]
  const uint8_t* k_pool;     // [NB][Hkv][bs][D]
  const uint8_t* v_pool;
  const float* k_scale;      // [NB][Hkv] (fp8 only)
  const float* v_scale;
  const int32_t* tables;     // [S][max_blocks]
  const int32_t* ctx_lens;   // [S]
  const int32_t* q_lens;     // [S]
  const int32_t* shared_blocks;  // [S] leading blocks other sequences also read (NULL: none)
  // Decode steps with the append taken into the decode launch (NULL otherwise):
  // row s's new K/V ([S][Hkv][D], pool element type) go to pool slot slots[s],
  // and the step attends to them for position ctx_lens[s] - 1 from here.
  const uint8_t* k_new;
  const uint8_t* v_new;
  const int32_t* slots;
  int32_t append_in_merge;   // with k_new: the merge launch, not the decode launch, stores them
  int32_t new_in_merge;      // with k_new (MFMA decode steps): the decode launch walks keys
                             // 0 .. L-2 and leaves partials for every row; the merge launch
                             // adds key L-1 from k_new / v_new
  int32_t kv_fp8;            // the pools hold fp8-e4m3 (k_new / v_new too)
  int32_t append_rows;       // with k_new in a step with prefill chunks: rows the prologue launch stores
  int32_t append_row_bytes;  // bytes of one (row, kv head) of k_new / v_new
  const int32_t* q_start;    // [S + 1] row offsets (NULL when every query_len is 1)
  const int32_t* row_seq;    // [Tq] sequence of each row (NULL when every query_len is 1)
  float* part_ml;            // [Tq][Hq][max_parts][2]  (m in log2 units, l)
  float* part_o;             // [Tq][Hq][max_parts][D]  unnormalised; float32, or
                             // bfloat16 (part_bf16: fp8 KV) in the first half
  int32_t part_bf16;
  const int32_t* chunk_entries;  // [chunk_capacity][2] (sequence, first column) of prefill tiles
  const int32_t* chunk_count;    // number of valid chunk entries (written by the prologue)
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t total_q;
  int32_t max_parts;         // partition slots per (row, head) in the partial buffers
  int32_t part_tokens;       // tokens per split-context partition of a decode row (multiple of 16)
  int32_t part_head;         // tokens a decode row's partition 0 is short by (multiple of 16, < part_tokens)
  int32_t chunk_part_tokens; // tokens per partition of a prefill-chunk row (multiple of 16)
  int32_t chunk_max_parts;   // partitions the chunk kernel walks per entry and kv head
  int32_t chunk_capacity;    // room for chunk entries in the workspace
  int32_t chunk_cols;        // (row, head) columns per chunk entry (chunk_entry_cols)
  int32_t small_q;           // sequences with query_len <= small_q run as decode items
  float scale_log2;          // softmax scale * log2(e)
};

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// two OCP E4M3FN bytes (the low or high 16 bits of w) -> two floats, hardware convert
template <bool HI>
__device__ __forceinline__ void fp8x2_to_f32(uint32_t w, float& a, float& b) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  a = v[0];
  b = v[1];
}

// A value every lane of the wave reads from the same address: readfirstlane
// tells the compiler it is uniform, so what is computed from it (block
// indices, buffer resources) stays in scalar registers.
__device__ __forceinline__ int uniform_load(const int32_t* ptr) {
  return __builtin_amdgcn_readfirstlane(*ptr);
}
// Split-context partition q of a row covers keys [part_begin, part_end) of
// its context: partitions of pt keys, the first h keys short (h = part_head
// for decode rows, 0 for prefill-chunk rows), so that the partitions a decode
// launch deals last (partition 0, which every row has) are the short ones.
__device__ __forceinline__ int part_begin(int q, int pt, int h) { return q == 0 ? 0 : q * pt - h; }
__device__ __forceinline__ int part_end(int q, int pt, int h) { return (q + 1) * pt - h; }
// partitions of a row whose partitions cover `keys` keys (none for none)
__device__ __forceinline__ int part_count(int keys, int pt, int h) {
  return keys > 0 ? (keys + h + pt - 1) / pt : 0;
}

// The split-context partition a decode launch's workgroup takes from its
// grid.y.  Partition q exists only for rows longer than q partitions, so the
// work per partition index falls as the index grows: dispatched last-first,
// the launch ends on partition 0, which every row has, and the chip stays
// filled to the end (dispatched first-first it ended on the few longest rows'
// last partitions, most slots idle).  Steps with a shared-prefix hint keep
// first-first, which measured faster for them.
__device__ __forceinline__ int dispatch_part(const StepParams& p) {
  return p.shared_blocks != nullptr ? (int)blockIdx.y : (int)(gridDim.y - 1 - blockIdx.y);
}

// An int that no running kernel writes, at an address every lane holds alike:
// read through the constant address space, so it is a scalar load whatever
// the kernel stores elsewhere (a vector load would be waited for together
// with every vector load in flight)
__device__ __forceinline__ int const_load(const int32_t* ptr) {
  return *(const __attribute__((address_space(4))) int32_t*)ptr;
}
// a pointer every lane holds alike, in scalar registers
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Buffer-resource loads of one K or V block.  The resource's record count
// covers the block's existing token rows only (0 for a block that counts no
// tokens: the clamped look-ahead past a wave's last block, an invalid table
// entry): an out-of-range buffer load returns zeros without touching memory,
// so those issue the same instructions with no branch and move no bytes.
// Word 3 is the gfx9-family untyped-buffer descriptor (32-bit data format).
constexpr int kBufferRsrcWord3 = 0x00020000;
typedef uint32_t u32x4_buf __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, kBufferRsrcWord3);
}

// NT sets the load's nontemporal hint (aux bit 1, value 2).  A K/V block that
// no other reader of the step touches is read exactly once: a nontemporal load
// (streaming policy) passes it by the caches.  On MI355X a random gather of
// 4 KiB runs moves ~6.85 TB/s this way against ~6.1 TB/s with ordinary loads
// -- but lines that other waves read again soon (a shared prefix, the four
// waves of a prefill tile) then come from HBM again, so those keep ordinary
// loads.
template <bool NT>
__device__ __forceinline__ uint4 load_block16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  const u32x4_buf v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, NT ? 2 : 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// s_waitcnt immediate (gfx9 fields): no vector memory and no LDS/scalar
// operation outstanding
constexpr int kWaitAll = 0x0070;

// Stores of split-context partials (unnormalised output rows), which the
// merge launch reads right after: with device scope (aux bit 4, sc1) rather
// than the default policy, which measured slower in the VALU decode launch.
constexpr int kPartialStore = 16;
__device__ __forceinline__ void store_partial(__amdgpu_buffer_rsrc_t r, int byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, kPartialStore);
}
__device__ __forceinline__ void store_partial(__amdgpu_buffer_rsrc_t r, int byte_off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, byte_off, 0, kPartialStore);
}

// unpack a 16-byte load of KV elements into floats (8 for 16-bit types, 16 for fp8)
template <int KV>
__device__ __forceinline__ void unpack16(const uint4& r, float* f) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  if constexpr (KV == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(w[i]); f[2 * i + 1] = bf16_hi(w[i]); }
  } else if constexpr (KV == kF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = f16_lo(w[i]); f[2 * i + 1] = f16_hi(w[i]); }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fp8x2_to_f32<false>(w[i], f[4 * i], f[4 * i + 1]);
      fp8x2_to_f32<true>(w[i], f[4 * i + 2], f[4 * i + 3]);
    }
  }
}

// 16-bit query/output element <-> float
template <int T>
__device__ __forceinline__ float load_q(const void* base, size_t idx) {
  const uint16_t u = reinterpret_cast<const uint16_t*>(base)[idx];
  if constexpr (T == kBF16) return __uint_as_float((uint32_t)u << 16);
  else return (float)__builtin_bit_cast(_Float16, u);
}

// float -> bfloat16 bits, round to nearest even (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32.  It agrees bit for bit with the add-0x7fff-plus-lsb
// rounding of the bit pattern (NaNs quieted, payload kept) on every
// sign / exponent / top-mantissa pattern with tie and tail variants.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// two floats -> two packed bfloat16 (a in the low half), one instruction
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <int T>
__device__ __forceinline__ uint16_t to_out_bits(float f) {
  if constexpr (T == kBF16) return f32_to_bf16_rne(f);
  else return __builtin_bit_cast(uint16_t, (_Float16)f);   // v_cvt_f16_f32, RNE
}

// ---------------------------------------------------------------------------
// wave64 cross-lane reductions
// ---------------------------------------------------------------------------
// DPP controls (gfx9): quad_perm, row_half_mirror, row_mirror
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// sum over aligned groups of N lanes (N in {1,2,4,8,16}); every lane gets its group's sum
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f<kDppQuadXor1>(v);
  if constexpr (N >= 4) v += dpp_f<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp_f<kDppRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f<kDppRowMirror>(v);
  return v;
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// {v[l], v[l ^ 16]} and {v[l], v[l ^ 32]} in lane-independent order (gfx950
// v_permlane16_swap / v_permlane32_swap: VALU, no LDS round trip), so both
// lanes of a pair compute the same max or sum.
__device__ __forceinline__ float max_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(p[0]), __int_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(p[0]), __int_as_float(p[1]));
}
// maximum over the 64 lanes of a fully active wave, in every lane
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppRowMirror>(v));
  return max_xor32(max_xor16(v));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(p[0]) + __int_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(p[0]) + __int_as_float(p[1]);
}
// sum over the 64 lanes of a fully active wave, in every lane (the same
// order of additions in every lane)
__device__ __forceinline__ float wave_sum(float v) {
  return sum_xor32(sum_xor16(group_sum<16>(v)));
}

}  // namespace pkv
