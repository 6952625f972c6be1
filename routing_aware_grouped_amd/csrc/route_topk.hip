// route_topk.hip -- step 1 of the layer: top-k routing, softmax weights and the
// per-local-expert token histogram.
//
// What is computed (RaMP arXiv 2604.26039, 2.1: the router sends each token to k of
// E experts; 2.3: the counts n_e of the GPU's experts sum to Bk; 3.2: the selection
// kernel counts this GPU's tokens per local expert in shared memory and ignores
// tokens routed elsewhere):
//   ids[t][0..k)  the k largest logits of token t, descending; equal logits go to
//                 the lower expert index and -0 equals +0
//   w[t][j]       softmax over the k chosen logits (renormalize = 1) or those
//                 experts' entries of the softmax over all E logits (renormalize = 0)
//   counts[e]     #{(t, j) : ids[t][j] = e0 + e},  e < E_loc
//
// Design (gfx950, wave64): a group of L lanes (L = 8..64, a power of two >= E when
// E <= 64, else 64) owns one token; lane i holds logits e = i, i + L, ... in
// registers as 64-bit order-preserving keys (float order in the high word, ~index in
// the low word, so one unsigned max also applies the lower-index tie rule).  Each of
// the k rounds is a register max plus a log2(L)-step butterfly of cross-lane
// shuffles; the winner's owner clears its key.  The histogram goes through LDS and
// then to global memory: with one workgroup the counts are stored directly; with
// many, a tiny kernel zeroes them first and workgroups add their LDS bins with
// global atomics (integer, so the result is exact and order-independent).
#include "moe_common.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 -> +0: the two compare equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_key_float(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o ^ 0x80000000u) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m, kWave);
  hi = __shfl_xor(hi, m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

template <int L>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

template <int L>
__device__ __forceinline__ float group_sum_f32(float v) {
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__global__ void zero_counts_kernel(int32_t* counts, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) counts[i] = 0;
}

// L lanes per token, MMAX >= ceil(E / L) logits per lane.
template <int L, int MMAX>
__global__ void __launch_bounds__(1024) route_topk_kernel(const float* __restrict__ logits, int32_t* __restrict__ ids,
                                  float* __restrict__ wout, int32_t* __restrict__ counts, int B,
                                  int E, int k, int e0, int E_loc, int renormalize,
                                  int single_wg) {
  extern __shared__ int32_t hist[];  // [E_loc]
  for (int i = threadIdx.x; i < E_loc; i += blockDim.x) hist[i] = 0;
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int gl = lane & (L - 1);  // lane inside the token group
  const int groups_per_wg = blockDim.x / L;
  const int group = threadIdx.x / L;
  const int M = (E + L - 1) / L;

  for (int t0 = blockIdx.x * groups_per_wg; t0 < B; t0 += gridDim.x * groups_per_wg) {
    const int t = t0 + group;
    const bool active = t < B;  // whole groups are inactive together
    uint64_t key[MMAX];
    const float* lrow = logits + (int64_t)(active ? t : 0) * E;
#pragma unroll
    for (int i = 0; i < MMAX; ++i) {
      const int e = gl + i * L;
      key[i] = 0;
      if (active && i < M && e < E)
        key[i] = ((uint64_t)float_order_key(lrow[e]) << 32) | (uint32_t)(~(uint32_t)e);
    }
    int my_id = -1;
    float my_logit = 0.f;
    float top = 0.f;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < MMAX; ++i) best = key[i] > best ? key[i] : best;
      best = group_max_u64<L>(best);
      const int e = (int)(~(uint32_t)best);
      const float lv = order_key_float((uint32_t)(best >> 32));
      if (j == 0) top = lv;
      if (gl == j) {
        my_id = e;
        my_logit = lv;
      }
      if ((e & (L - 1)) == gl) {
        const int slot = e / L;
#pragma unroll
        for (int i = 0; i < MMAX; ++i)
          if (i == slot) key[i] = 0;
      }
    }
    // weights
    float ex = (gl < k) ? expf(my_logit - top) : 0.f;
    float den;
    if (renormalize) {
      den = group_sum_f32<L>(ex);
    } else {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < MMAX; ++i) {
        const int e = gl + i * L;
        if (active && i < M && e < E) part += expf(lrow[e] - top);
      }
      den = group_sum_f32<L>(part);
    }
    if (active && gl < k) {
      ids[(int64_t)t * k + gl] = my_id;
      wout[(int64_t)t * k + gl] = ex / den;
      const int le = my_id - e0;
      if (le >= 0 && le < E_loc) atomicAdd(&hist[le], 1);
    }
  }
  __syncthreads();
  if (single_wg) {
    for (int i = threadIdx.x; i < E_loc; i += blockDim.x) counts[i] = hist[i];
  } else {
    for (int i = threadIdx.x; i < E_loc; i += blockDim.x)
      if (hist[i]) atomicAdd(&counts[i], hist[i]);
  }
}

template <int L, int MMAX>
hipError_t launch_lm(const moe_problem& p, const float* logits, int32_t* ids, float* w,
                     int32_t* counts, hipStream_t s) {
  const int B = p.tokens;
  // one 1024-thread workgroup for small batches (no zeroing launch needed),
  // otherwise 256-thread workgroups over the token range
  const int groups_single = 1024 / L;
  const bool single = B <= 4 * groups_single;
  const int threads = single ? 1024 : 256;
  int grid = 1;
  if (!single) {
    const int groups = threads / L;
    grid = (B + groups - 1) / groups;
    if (grid > 4096) grid = 4096;
    zero_counts_kernel<<<(p.local_experts + 255) / 256, 256, 0, s>>>(counts, p.local_experts);
  }
  route_topk_kernel<L, MMAX><<<grid, threads, p.local_experts * sizeof(int32_t), s>>>(
      logits, ids, w, counts, B, p.num_experts, p.top_k, p.expert_begin, p.local_experts,
      p.renormalize, single ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_topk(const moe_problem& p, const float* logits, int32_t* ids, float* w,
                             int32_t* counts, hipStream_t s) {
  const int E = p.num_experts;
  if (E <= 8) return launch_lm<8, 1>(p, logits, ids, w, counts, s);
  if (E <= 16) return launch_lm<16, 1>(p, logits, ids, w, counts, s);
  if (E <= 32) return launch_lm<32, 1>(p, logits, ids, w, counts, s);
  if (E <= 64) return launch_lm<64, 1>(p, logits, ids, w, counts, s);
  if (E <= 128) return launch_lm<64, 2>(p, logits, ids, w, counts, s);
  if (E <= 256) return launch_lm<64, 4>(p, logits, ids, w, counts, s);
  if (E <= 512) return launch_lm<64, 8>(p, logits, ids, w, counts, s);
  if (E <= 1024) return launch_lm<64, 16>(p, logits, ids, w, counts, s);
  return launch_lm<64, 64>(p, logits, ids, w, counts, s);
}

}  // namespace moe
