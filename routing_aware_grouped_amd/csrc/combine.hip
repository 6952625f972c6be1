// combine.hip -- step 5: the router-weighted combine.
//
// GC-MoE (arXiv 2611.04222) 2.1 Eq. 1 sums each token's routed expert outputs with
// its routing weights g_{t,j}; its combine role accumulates the valid top-k slots
// in fp32 in slot order and packs to bf16.  Here:
//   y[t] = sum_{j = 0..k-1, slot_pos[t*k+j] >= 0} w[t][j] * y_slots[slot_pos[t*k+j]]
// in fp32 in ascending j, rounded once to the output dtype; tokens whose experts are
// all on other GPUs get zeros.  Gather form (each token reads its own k rows), so
// the result is deterministic without atomics.
//
// Design: one workgroup per token (grid-stride), 16-byte vector loads and stores
// along H; the token's slot rows and weights are workgroup-uniform (scalar loads).
#include "moe_common.h"

namespace moe {
namespace {

template <bool F32>
__global__ void __launch_bounds__(256)
combine_kernel(const void* __restrict__ y_slots, const int32_t* __restrict__ slot_pos,
               const float* __restrict__ w, void* __restrict__ y, int B, int H, int k,
               int64_t rows_max) {
  constexpr int VEC = F32 ? 4 : 8;  // elements per 16-byte vector
  for (int t = blockIdx.x; t < B; t += gridDim.x) {
    for (int h0 = threadIdx.x * VEC; h0 < H; h0 += blockDim.x * VEC) {
      float acc[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
      for (int j = 0; j < k; ++j) {
        const int pos = slot_pos[(int64_t)t * k + j];
        if (pos < 0 || pos >= rows_max) continue;
        const float g = w[(int64_t)t * k + j];
        if (F32) {
          const f32x4 v = *(const f32x4*)((const float*)y_slots + (int64_t)pos * H + h0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(g, v[i], acc[i]);
        } else {
          const u32x4 v = *(const u32x4*)((const uint16_t*)y_slots + (int64_t)pos * H + h0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] = __builtin_fmaf(g, __uint_as_float(v[i] << 16), acc[2 * i]);
            acc[2 * i + 1] = __builtin_fmaf(g, __uint_as_float(v[i] & 0xFFFF0000u), acc[2 * i + 1]);
          }
        }
      }
      if (F32) {
        f32x4 o = {acc[0], acc[1], acc[2], acc[3]};
        *(f32x4*)((float*)y + (int64_t)t * H + h0) = o;
      } else {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
        *(u32x4*)((uint16_t*)y + (int64_t)t * H + h0) = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const moe_problem& p, const void* y_slots, const int32_t* slot_pos,
                          const float* w, void* y, int64_t rows_max, hipStream_t s) {
  int grid = p.tokens < 4096 ? p.tokens : 4096;
  if (p.act_dtype == MOE_F32)
    combine_kernel<true><<<grid, 256, 0, s>>>(y_slots, slot_pos, w, y, p.tokens, p.hidden, p.top_k, rows_max);
  else
    combine_kernel<false><<<grid, 256, 0, s>>>(y_slots, slot_pos, w, y, p.tokens, p.hidden, p.top_k, rows_max);
  return hipGetLastError();
}

}  // namespace moe
