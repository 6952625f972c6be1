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
// Shared experts (GC-MoE section 4: their output is one more lane of the combine):
// after the k routed lanes, lane k + i adds shared expert i's row of y_slots with
// weight 1; those rows follow the routed ones, in token order, ceil(B / b) row-
// blocks per shared expert (b = BLOCK_M of the chosen configuration, read with the
// routed row-block count from device memory).  A configuration outside the menu
// means the grouped FFN ran no tile, and the shared lanes then add nothing.
//
// Design: a workgroup takes one token and a chunk of 256 16-byte vectors along H
// (grid-stride over tokens x chunks, so a small batch still spreads over many
// workgroups).  The token's slot rows and weights are read once into LDS; each
// thread then issues the loads of up to 8 slot rows before it adds them, so the
// k row reads overlap instead of waiting one after another.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kCombineThreads = 256;
constexpr int kCombineBatch = 8;  // slot rows loaded before they are added

template <bool F32>
__global__ void __launch_bounds__(kCombineThreads)
combine_kernel(const void* __restrict__ y_slots, const int32_t* __restrict__ slot_pos,
               const float* __restrict__ w, void* __restrict__ y, int B, int H, int k,
               int64_t rows_max, int chunks, int cw, int n_shared,
               const int32_t* __restrict__ num_blocks,
               const int32_t* __restrict__ variant) {
  constexpr int VEC = F32 ? 4 : 8;  // elements per 16-byte vector
  __shared__ int s_pos[32 + kMaxShared];
  __shared__ float s_w[32 + kMaxShared];
  // first row of the shared experts' rows and the rows per shared expert
  int64_t sh0 = 0, shn = 0;
  if (n_shared > 0) {
    const int v = *variant;
    const int nb = *num_blocks;
    if (v >= 0 && v < kNumVariants && nb >= 0) {
      const int bm = kVariants[v].bm;
      sh0 = (int64_t)nb * bm;
      shn = (int64_t)((B + bm - 1) / bm) * bm;
    } else {
      n_shared = 0;
    }
  }
  const int lanes = k + n_shared;
  const int64_t items = (int64_t)B * chunks;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int t = (int)(item / chunks);
    const int c = (int)(item - (int64_t)t * chunks);
    __syncthreads();  // the previous item's readers are done with s_pos / s_w
    if (threadIdx.x < k) {
      const int pos = slot_pos[(int64_t)t * k + threadIdx.x];
      s_pos[threadIdx.x] = (pos < 0 || pos >= rows_max) ? -1 : pos;
      s_w[threadIdx.x] = w[(int64_t)t * k + threadIdx.x];
    } else if (threadIdx.x < lanes) {  // shared expert lanes, weight 1
      const int64_t row = sh0 + (threadIdx.x - k) * shn + t;
      s_pos[threadIdx.x] = row < rows_max ? (int)row : -1;
      s_w[threadIdx.x] = 1.0f;
    }
    __syncthreads();
    const int hend = (c + 1) * cw < H ? (c + 1) * cw : H;  // this item's columns [c cw, hend)
    for (int h0 = c * cw + (int)threadIdx.x * VEC; h0 < hend; h0 += kCombineThreads * VEC) {
      float acc[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
      for (int j0 = 0; j0 < lanes; j0 += kCombineBatch) {
        u32x4 v[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
          const int pos = j0 + u < lanes ? s_pos[j0 + u] : -1;
          const char* src = (const char*)y_slots + ((int64_t)pos * H + h0) * (F32 ? 4 : 2);
          v[u] = pos >= 0 ? *(const u32x4*)src : u32x4{0u, 0u, 0u, 0u};
        }
        // accumulated in ascending j, in fp32
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
          if (j0 + u >= lanes || s_pos[j0 + u] < 0) continue;
          const float g = s_w[j0 + u];
          if (F32) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[i] = __builtin_fmaf(g, __uint_as_float(v[u][i]), acc[i]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              acc[2 * i] = __builtin_fmaf(g, __uint_as_float(v[u][i] << 16), acc[2 * i]);
              acc[2 * i + 1] =
                  __builtin_fmaf(g, __uint_as_float(v[u][i] & 0xFFFF0000u), acc[2 * i + 1]);
            }
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
                          const float* w, const int32_t* num_blocks, const int32_t* variant,
                          void* y, int64_t rows_max, hipStream_t s) {
  const int n_shared = num_blocks && variant ? p.shared_experts : 0;
  // a small batch splits each token's columns over workgroups (2048 bf16 columns
  // per item); a large one gives each workgroup whole tokens
  const int vec = p.act_dtype == MOE_F32 ? 4 : 8;
  const int span = kCombineThreads * vec;
  const int chunks = p.tokens >= 512 ? 1 : (p.hidden + span - 1) / span;
  const int cw = (p.hidden + chunks * span - 1) / (chunks * span) * span;
  const int64_t items = (int64_t)p.tokens * chunks;
  const int grid = items < 4096 ? (int)items : 4096;
  if (p.act_dtype == MOE_F32)
    combine_kernel<true><<<grid, kCombineThreads, 0, s>>>(y_slots, slot_pos, w, y, p.tokens,
                                                          p.hidden, p.top_k, rows_max, chunks, cw,
                                                          n_shared, num_blocks, variant);
  else
    combine_kernel<false><<<grid, kCombineThreads, 0, s>>>(y_slots, slot_pos, w, y, p.tokens,
                                                           p.hidden, p.top_k, rows_max, chunks, cw,
                                                           n_shared, num_blocks, variant);
  return hipGetLastError();
}

}  // namespace moe
