// Copy-on-write on the device: copy whole blocks (every kv head, every slot)
// of the K and V pools, and their fp8 scales, from source to destination ids.
//
// Page "Serving LLMs with vLLM: Continuous Batching and PagedAttention
// Explained", section "Copy-on-Write": before a sequence writes into a block
// other tables still point at, the block is copied to a fresh one and only the
// writer's table is changed.  The host block manager decides the pairs; this
// kernel moves the bytes, 16 at a time.
#include "../../include/pagedkv_blocks.h"
#include "pkv_launch.h"

namespace pkv {

// threads ordered (pair, K|V, piece) with the 16-byte piece fastest
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ k_pool,
                                                          uint8_t* __restrict__ v_pool,
                                                          float* __restrict__ k_scale,
                                                          float* __restrict__ v_scale,
                                                          const int32_t* __restrict__ pairs,
                                                          int32_t num_pairs, int32_t num_blocks,
                                                          int64_t pieces_per_block,
                                                          int32_t num_kv_heads) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_pair = 2 * pieces_per_block;
  if (i >= (int64_t)num_pairs * per_pair) return;
  const int32_t pr = (int32_t)(i / per_pair);
  const int64_t r = i - (int64_t)pr * per_pair;
  const bool is_v = r >= pieces_per_block;
  const int64_t piece = is_v ? r - pieces_per_block : r;
  const int32_t src = pairs[2 * pr];
  const int32_t dst = pairs[2 * pr + 1];
  if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) return;
  uint4* pool = reinterpret_cast<uint4*>(is_v ? v_pool : k_pool);
  pool[(int64_t)dst * pieces_per_block + piece] = pool[(int64_t)src * pieces_per_block + piece];
  float* sc = is_v ? v_scale : k_scale;
  if (sc != nullptr && piece < num_kv_heads)
    sc[(int64_t)dst * num_kv_heads + piece] = sc[(int64_t)src * num_kv_heads + piece];
}

}  // namespace pkv

extern "C" int paged_kv_copy_blocks(const pkv_pool* pool, void* k_pool, void* v_pool,
                                    float* k_scale, float* v_scale, const int32_t* pairs,
                                    int32_t num_pairs, void* stream) {
  if (pool == nullptr) return PKV_ERR_NULL;
  if (pool->num_blocks < 1 || pool->num_kv_heads < 1 || pool->block_size < 1 || pool->head_dim < 1)
    return PKV_ERR_SHAPE;
  if (pool->kv_dtype != PKV_F16 && pool->kv_dtype != PKV_BF16 && pool->kv_dtype != PKV_FP8_E4M3)
    return PKV_ERR_DTYPE;
  if (num_pairs < 0) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !pairs) return PKV_ERR_NULL;
  if (pool->kv_dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) return PKV_ERR_NULL;
  const int64_t block_bytes = (int64_t)pool->num_kv_heads * pool->block_size * pool->head_dim *
                              (pool->kv_dtype == PKV_FP8_E4M3 ? 1 : 2);
  if (block_bytes % 16 != 0 || ((uintptr_t)k_pool & 15) || ((uintptr_t)v_pool & 15))
    return PKV_ERR_SHAPE;
  const int64_t pieces = block_bytes / 16;
  const int64_t threads = (int64_t)num_pairs * 2 * pieces;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return PKV_ERR_SHAPE;
  (void)hipGetLastError();   // drop an error some earlier, unrelated call left behind
  hipLaunchKernelGGL(pkv::copy_blocks_kernel, dim3((uint32_t)blocks), dim3(256), 0,
                     (hipStream_t)stream, (uint8_t*)k_pool, (uint8_t*)v_pool, k_scale, v_scale,
                     pairs, num_pairs, pool->num_blocks, pieces, pool->num_kv_heads);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
