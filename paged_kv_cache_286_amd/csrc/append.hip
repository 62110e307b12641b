// KV append: copy this step's new K/V rows into their pool slots.
//
// Page "Serving LLMs with vLLM: Continuous Batching and PagedAttention
// Explained", section "Growing During Decode": a decode step writes the new
// token into the next slot of the sequence's last block.  The host names the
// slot of every new row (slot = block * block_size + offset); the kernel is a
// pure scatter of 16-byte pieces, bit for bit.
#include "pkv_launch.h"

namespace pkv {

// One thread moves one 16-byte piece.  Threads are ordered (K|V, row, head,
// piece) with the piece fastest, so a wave reads and writes whole contiguous
// (row, head) runs.
__global__ __launch_bounds__(256) void kv_append_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, int32_t num_tokens, int32_t num_kv_heads,
    int32_t pieces_per_head, int32_t head_bytes, int32_t block_size, int64_t num_slots) {
  const int64_t per_side = (int64_t)num_tokens * num_kv_heads * pieces_per_head;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= 2 * per_side) return;
  const bool is_v = i >= per_side;
  const int64_t r = is_v ? i - per_side : i;
  const int64_t hp = (int64_t)num_kv_heads * pieces_per_head;
  const int32_t token = (int32_t)(r / hp);
  const int32_t rem = (int32_t)(r - (int64_t)token * hp);
  const int32_t head = rem / pieces_per_head;
  const int32_t piece = rem - head * pieces_per_head;
  const int32_t slot = slots[token];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  const int32_t blk = slot / block_size;
  const int32_t off = slot - blk * block_size;
  const size_t dst = (((size_t)blk * num_kv_heads + head) * block_size + off) * (size_t)head_bytes +
                     (size_t)piece * 16;
  const size_t src = ((size_t)token * num_kv_heads + head) * (size_t)head_bytes + (size_t)piece * 16;
  const uint4 val = *reinterpret_cast<const uint4*>((is_v ? v_new : k_new) + src);
  *reinterpret_cast<uint4*>((is_v ? v_pool : k_pool) + dst) = val;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const int32_t head_bytes = a.head_dim * a.elem_bytes;
  const int32_t pieces = head_bytes / 16;
  const int64_t threads = 2LL * a.num_tokens * a.num_kv_heads * pieces;
  if (threads == 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  (void)hipGetLastError();   // drop an error some earlier, unrelated call left behind
  hipLaunchKernelGGL(kv_append_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     (uint8_t*)a.k_pool, (uint8_t*)a.v_pool, (const uint8_t*)a.k_new,
                     (const uint8_t*)a.v_new, a.slots, a.num_tokens, a.num_kv_heads, pieces,
                     head_bytes, a.block_size, (int64_t)a.num_blocks * a.block_size);
  return hipGetLastError();
}

}  // namespace pkv
