// fused_ffn.h -- host launchers of the fused small-batch plan (fused_ffn.hip).
// Internal header of the GPU library (not part of the C ABI).
#pragma once

#include "moe_common.h"

namespace moe {

// The fused plan for small batches (fused_ffn.hip): the size of its workspace (a 256-byte header holding the device status word,
// then the fp32 slice partials [I / slice][B k][H]), the one FFN launch, and the
// combine that adds the slices.
int64_t fused_ws_bytes(const moe_problem& p);
hipError_t launch_fused_ffn(const moe_problem& p, const void* x, const void* w1, const void* w3,
                            const void* w2, const float* s1, const float* s3, const float* s2,
                            const int32_t* sorted_slots, const int32_t* block_expert,
                            const int32_t* num_blocks, const int32_t* variant, void* ws,
                            int num_cus, int64_t rows_max, hipStream_t s);
hipError_t launch_combine_fused(const moe_problem& p, const void* ws, const int32_t* slot_pos,
                                const float* w, void* y, hipStream_t s);

}  // namespace moe
