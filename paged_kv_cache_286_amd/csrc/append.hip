// KV append: copy this step's new K/V rows into their pool slots.
//
// Page "Serving LLMs with vLLM: Continuous Batching and PagedAttention
// Explained", section "Growing During Decode": a decode step writes the new
// token into the next slot of the sequence's last block.  The host names the
// slot of every new row (slot = block * block_size + offset); the kernel is a
// pure scatter of 16-byte pieces, bit for bit.
#include "pkv_launch.h"

namespace pkv {

// One workgroup per (row, K|V): the row's slot is read once (a scalar load),
// and the threads move its (head, piece) 16-byte pieces with the piece
// fastest, so a wave reads and writes whole contiguous (row, head) runs.
// pieces_per_head is a power of two (head_bytes / 16 with head_dim 64 or 128).
__global__ __launch_bounds__(256) void kv_append_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, int32_t num_kv_heads, int32_t piece_shift,
    int32_t head_bytes, int32_t block_size, int64_t num_slots) {
  const int32_t token = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const int32_t slot = slots[token];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  const int32_t blk = slot / block_size;
  const int32_t off = slot - blk * block_size;
  const uint8_t* src = (is_v ? v_new : k_new) + (size_t)token * num_kv_heads * head_bytes;
  uint8_t* dst = (is_v ? v_pool : k_pool) + ((size_t)blk * num_kv_heads * block_size + off) * head_bytes;
  const int32_t pieces = num_kv_heads << piece_shift;
  for (int32_t j = threadIdx.x; j < pieces; j += blockDim.x) {
    const int32_t head = j >> piece_shift;
    const int32_t piece = j - (head << piece_shift);
    const uint4 val = *reinterpret_cast<const uint4*>(src + (size_t)j * 16);
    *reinterpret_cast<uint4*>(dst + ((size_t)head * block_size * head_bytes + (size_t)piece * 16)) = val;
  }
}

// ---------------------------------------------------------------------------
// quantising append: 16-bit rows into an fp8-e4m3 pool
// ---------------------------------------------------------------------------
// float -> OCP E4M3FN byte: round to nearest, ties to even, saturate at +-448,
// NaN -> 0x7F.  Below 2^-6 the format is evenly spaced by 2^-9, so the code is
// rint(a * 2^9) (0 .. 8, and 8 is the first normal code); above, a value in
// [2^E, 2^(E+1)) is rint(a * 2^(3-E)) eighths of 2^E (8 .. 16, 16 carrying
// into the next exponent).  Both scalings are exact, so rint is the only
// rounding.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return 0x7Fu;
  if (a >= 448.f) return sign | 0x7Eu;
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.f);
  } else {
    int e;
    (void)frexpf(a, &e);                 // a = f * 2^e, f in [0.5, 1)
    int E = e - 1;
    int m = (int)rintf(ldexpf(a, 3 - E)) - 8;
    if (m == 8) { E += 1; m = 0; }
    code = (uint32_t)(((E + 7) << 3) | m);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// blocks whose slot 0 is written take the caller's per-head scale
__global__ __launch_bounds__(256) void kv_append_scale_init_kernel(
    float* __restrict__ k_scale, float* __restrict__ v_scale, const float* __restrict__ k_init,
    const float* __restrict__ v_init, const int32_t* __restrict__ slots, int32_t num_tokens,
    int32_t num_kv_heads, int32_t block_size, int64_t num_slots) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)num_tokens * num_kv_heads) return;
  const int32_t token = (int32_t)(i / num_kv_heads);
  const int32_t head = (int32_t)(i - (int64_t)token * num_kv_heads);
  const int32_t slot = slots[token];
  if (slot < 0 || (int64_t)slot >= num_slots || slot % block_size != 0) return;
  const int64_t idx = (int64_t)(slot / block_size) * num_kv_heads + head;
  k_scale[idx] = k_init[head];
  v_scale[idx] = v_init[head];
}

// one thread: 16 values of one (row, head) -> 16 fp8 bytes, divided (IEEE
// float32) by the scale of the destination block and head
template <int NT>
__global__ __launch_bounds__(256) void kv_append_quant_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const int32_t* __restrict__ slots, int32_t num_tokens,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_slots) {
  const int32_t pieces = head_dim / 16;
  const int64_t per_side = (int64_t)num_tokens * num_kv_heads * pieces;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= 2 * per_side) return;
  const bool is_v = i >= per_side;
  const int64_t r = is_v ? i - per_side : i;
  const int64_t hp = (int64_t)num_kv_heads * pieces;
  const int32_t token = (int32_t)(r / hp);
  const int32_t rem = (int32_t)(r - (int64_t)token * hp);
  const int32_t head = rem / pieces;
  const int32_t piece = rem - head * pieces;
  const int32_t slot = slots[token];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  const int32_t blk = slot / block_size;
  const int32_t off = slot - blk * block_size;
  const float sc = (is_v ? v_scale : k_scale)[(int64_t)blk * num_kv_heads + head];
  const uint16_t* src = (is_v ? v_new : k_new) + ((int64_t)token * num_kv_heads + head) * head_dim + piece * 16;
  const uint4 w0 = reinterpret_cast<const uint4*>(src)[0];
  const uint4 w1 = reinterpret_cast<const uint4*>(src)[1];
  float f[16];
  unpack16<NT>(w0, f);
  unpack16<NT>(w1, f + 8);
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 16; ++e) out[e / 4] |= f32_to_e4m3_sat(__fdiv_rn(f[e], sc)) << (8 * (e % 4));
  uint8_t* dst = (is_v ? v_pool : k_pool) +
                 (((int64_t)blk * num_kv_heads + head) * block_size + off) * head_dim + piece * 16;
  *reinterpret_cast<uint4*>(dst) = make_uint4(out[0], out[1], out[2], out[3]);
}

hipError_t launch_append_quant(const AppendArgs& a, int new_dtype, float* k_scale, float* v_scale,
                               const float* k_init, const float* v_init, hipStream_t stream) {
  const int64_t num_slots = (int64_t)a.num_blocks * a.block_size;
  (void)hipGetLastError();   // drop an error some earlier, unrelated call left behind
  if (k_init != nullptr) {
    const int64_t n = (int64_t)a.num_tokens * a.num_kv_heads;
    hipLaunchKernelGGL(kv_append_scale_init_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0,
                       stream, k_scale, v_scale, k_init, v_init, a.slots, a.num_tokens,
                       a.num_kv_heads, a.block_size, num_slots);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t threads = 2LL * a.num_tokens * a.num_kv_heads * (a.head_dim / 16);
  const dim3 grid((uint32_t)((threads + 255) / 256));
  if (new_dtype == kBF16)
    hipLaunchKernelGGL((kv_append_quant_kernel<kBF16>), grid, dim3(256), 0, stream,
                       (uint8_t*)a.k_pool, (uint8_t*)a.v_pool, k_scale, v_scale,
                       (const uint16_t*)a.k_new, (const uint16_t*)a.v_new, a.slots, a.num_tokens,
                       a.num_kv_heads, a.head_dim, a.block_size, num_slots);
  else
    hipLaunchKernelGGL((kv_append_quant_kernel<kF16>), grid, dim3(256), 0, stream,
                       (uint8_t*)a.k_pool, (uint8_t*)a.v_pool, k_scale, v_scale,
                       (const uint16_t*)a.k_new, (const uint16_t*)a.v_new, a.slots, a.num_tokens,
                       a.num_kv_heads, a.head_dim, a.block_size, num_slots);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const int32_t head_bytes = a.head_dim * a.elem_bytes;
  const int32_t pieces = head_bytes / 16;
  int32_t shift = 0;
  while ((1 << shift) < pieces) ++shift;
  if ((1 << shift) != pieces || head_bytes % 16 != 0) return hipErrorInvalidValue;
  if (a.num_tokens == 0) return hipSuccess;
  (void)hipGetLastError();   // drop an error some earlier, unrelated call left behind
  hipLaunchKernelGGL(kv_append_kernel, dim3((uint32_t)a.num_tokens, 2), dim3(256), 0, stream,
                     (uint8_t*)a.k_pool, (uint8_t*)a.v_pool, (const uint8_t*)a.k_new,
                     (const uint8_t*)a.v_new, a.slots, a.num_kv_heads, shift, head_bytes,
                     a.block_size, (int64_t)a.num_blocks * a.block_size);
  return hipGetLastError();
}

}  // namespace pkv
