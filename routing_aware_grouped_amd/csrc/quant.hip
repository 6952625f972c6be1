// quant.hip -- FP8 E4M3FN quantization of the activations, per token and per
// group of 128 hidden columns (the 1 x 128 activation scaling that goes with the
// 128 x 128 weight blocks of DeepSeek-V3's FP8 recipe, which RaMP (arXiv
// 2604.26039) section 3.3 and appendix A.8 use for both expert GEMMs):
//   s = amax / 448,  q = E4M3FN(clamp(x / s, -448, 448)),  x ~ q * s.
//
// The same quantization serves h before the down GEMM (RaMP appendix A.8
// quantizes the gated activation to FP8): there the rows are the padded slot rows
// of the expert grouping, their count comes from device memory (the chosen
// configuration's BLOCK_M times the row-block count, then the shared experts' rows,
// ceil(B / BLOCK_M) row-blocks each, tokens in order) and padding rows are skipped.
//
// Design: one group (128 bf16 = 256 bytes) per 16 lanes, each lane holding one
// 16-byte chunk of 8 values; the group maximum is a 16-lane xor-shuffle
// reduction; a 256-thread workgroup covers 16 groups.  fp32 division is the
// correctly rounded one (HIP's default), and the hardware conversion rounds to
// nearest even, so the codes match a plain CPU implementation bit for bit.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kGroupsPerWg = kQuantThreads / 16;

// PADDED: rows are slot rows of h; only rows r < num_blocks * BLOCK_M of the chosen
// configuration with sorted_slots[r] >= 0 are quantized
template <bool PADDED>
__global__ void __launch_bounds__(kQuantThreads)
quant_act_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ s,
                 int64_t ngroups, int G, const int32_t* __restrict__ sorted_slots,
                 const int32_t* __restrict__ num_blocks, const int32_t* __restrict__ variant,
                 int B, int n_shared) {
  const int l16 = threadIdx.x & 15;
  int64_t routed = 0, shn = 1;  // routed rows; rows per shared expert
  if constexpr (PADDED) {
    const int v = *variant;
    const int64_t nb = *num_blocks;
    int64_t rows = 0;
    if (v >= 0 && v < kNumVariants && nb >= 0) {
      const int bm = kVariants[v].bm;
      routed = nb * bm;
      shn = (int64_t)((B + bm - 1) / bm) * bm;
      rows = routed + n_shared * shn;
    }
    ngroups = rows * G < ngroups ? rows * G : ngroups;
  }
  // 16 consecutive lanes share a group, so a group's lanes are always all
  // active together (the shuffles below stay inside the 16 lanes)
  for (int64_t grp = (int64_t)blockIdx.x * kGroupsPerWg + (threadIdx.x >> 4); grp < ngroups;
       grp += (int64_t)gridDim.x * kGroupsPerWg) {
    const int64_t t = grp / G;
    const int g = (int)(grp - t * G);
    if constexpr (PADDED) {  // padding rows are skipped (uniform over the 16 lanes)
      if (t < routed ? sorted_slots[t] < 0 : (t - routed) % shn >= B) continue;
    }
    const int64_t off = (t * G + g) * 128 + l16 * 8;  // = t * H + 128 g + 8 l16
    const u32x4 v = *(const u32x4*)(x + off);
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
    const float sc = amax / 448.0f;
    u32x2 o;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      float c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = amax > 0.f ? f[4 * w + i] / sc : 0.f;
        c[i] = fminf(fmaxf(r, -448.0f), 448.0f);
      }
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], p, true);
      o[w] = (uint32_t)p;
    }
    *(u32x2*)(q + off) = o;
    if (l16 == 0) s[grp] = sc;
  }
}

}  // namespace

hipError_t launch_quant_act(const moe_problem& p, const void* x, uint8_t* xq, float* xs,
                            hipStream_t s) {
  const int G = p.hidden / 128;
  const int64_t ngroups = (int64_t)p.tokens * G;
  int64_t grid = (ngroups + kGroupsPerWg - 1) / kGroupsPerWg;
  if (grid > 4096) grid = 4096;
  quant_act_kernel<false><<<(int)grid, kQuantThreads, 0, s>>>((const uint16_t*)x, xq, xs, ngroups,
                                                               G, nullptr, nullptr, nullptr, 0, 0);
  return hipGetLastError();
}

hipError_t launch_quant_h(const moe_problem& p, const void* h, uint8_t* hq, float* hs,
                          const int32_t* sorted_slots, const int32_t* num_blocks,
                          const int32_t* variant, int64_t rows_max, hipStream_t s) {
  const int G = p.inter / 128;
  const int64_t ngroups = rows_max * G;  // the device count bounds it further
  int64_t grid = (ngroups + kGroupsPerWg - 1) / kGroupsPerWg;
  if (grid > 4096) grid = 4096;
  quant_act_kernel<true><<<(int)grid, kQuantThreads, 0, s>>>((const uint16_t*)h, hq, hs, ngroups,
                                                              G, sorted_slots, num_blocks, variant,
                                                              p.tokens, p.shared_experts);
  return hipGetLastError();
}

}  // namespace moe
