// Host-side launch interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"

namespace pkv {

struct AppendArgs {
  void* k_pool;
  void* v_pool;
  const void* k_new;
  const void* v_new;
  const int32_t* slots;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t elem_bytes;
  int32_t block_size;
  int32_t num_blocks;
};

// one step's launch plan, fixed from host scalars only
struct StepPlan {
  int32_t kv_dtype;
  int32_t q_dtype;
  int32_t head_dim;
  int32_t group;          // query heads per kv head
  int32_t heads_per_wg;   // query heads one VALU decode workgroup handles
  bool decode_on_mfma;    // decode rows run on the MFMA tile kernel instead of the VALU kernel
  int32_t chunk_grid;     // workgroups of the chunk kernel (0: no sequence has query_len > 1)
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_append_quant(const AppendArgs& a, int new_dtype, float* k_scale, float* v_scale,
                               const float* k_init, const float* v_init, hipStream_t stream);
hipError_t launch_prologue(const StepParams& p, hipStream_t stream);
hipError_t launch_check(const StepParams& p, int32_t* record, int32_t max_ctx, int32_t max_q,
                        hipStream_t stream);
hipError_t launch_decode(const StepParams& p, const StepPlan& plan, hipStream_t stream);
hipError_t launch_decode_mfma(const StepParams& p, const StepPlan& plan, hipStream_t stream);
hipError_t launch_step_mfma(const StepParams& p, const StepPlan& plan, hipStream_t stream);
hipError_t launch_reduce(const StepParams& p, const StepPlan& plan, hipStream_t stream);
bool decode_supported(const StepPlan& plan);

}  // namespace pkv
