// select_config.hip -- step 2: the on-GPU cost model that picks the tile
// configuration from the live per-expert histogram.
//
// RaMP (arXiv 2604.26039) 2.2 Eq. 1 gives the tiles and waves of configuration c on
// load n: T_c = q_c * sum_e ceil(n_e / b_c), W_c = ceil(T_c / S_c); 3.1 Eq. 3 predicts
// t_c = th_c0 + th_c1 W_c + th_c2 T_c + th_c3 A(n); 2.4 Eq. 2 takes the argmin.  The
// grouped kernel here runs two phases (gate/up, then down), so T and W sum over
// the phases: T = (q1 + q2) rt, W = ceil(q1 rt / S1) + ceil(q2 rt / S2) with
// rt = sum_e ceil(n_e / b).  A(n) is read as the number of active experts
// (n_e > 0), the term the appendix A.1 discussion says sets the floor at small
// loads.  The prediction is one fp32 FMA chain,
//   t = fma(th3, A, fma(th2, T, fma(th1, W, th0))),
// and the first index wins ties.  One workgroup; one wave per configuration
// (3.2: one warp per menu entry) reduces its row-tile count with cross-lane adds.
#include "moe_common.h"

namespace moe {
namespace {

__global__ void select_config_kernel(const int32_t* __restrict__ counts, int E_loc,
                                     const float* __restrict__ theta, CostTable tab,
                                     int32_t* __restrict__ variant, float* __restrict__ t_hat) {
  __shared__ float tv[kNumVariants];
  __shared__ int active;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  if (threadIdx.x == 0) active = 0;
  __syncthreads();
  if (wave == 0) {
    int a = 0;
    for (int e = lane; e < E_loc; e += kWave) a += counts[e] > 0;
    for (int m = 32; m >= 1; m >>= 1) a += __shfl_xor(a, m, kWave);
    if (lane == 0) active = a;
  }
  __syncthreads();
  for (int v = wave; v < kNumVariants; v += nwaves) {
    const int b = tab.b[v];
    int rt = 0;
    for (int e = lane; e < E_loc; e += kWave) rt += (counts[e] + b - 1) / b;
    for (int m = 32; m >= 1; m >>= 1) rt += __shfl_xor(rt, m, kWave);
    if (lane == 0) {
      const int T1 = tab.q1[v] * rt, T2 = tab.q2[v] * rt;
      const int W = (T1 + tab.S1[v] - 1) / tab.S1[v] + (T2 + tab.S2[v] - 1) / tab.S2[v];
      const int T = T1 + T2;
      const float* th = theta + 4 * v;
      const float t = __builtin_fmaf(
          th[3], (float)active, __builtin_fmaf(th[2], (float)T, __builtin_fmaf(th[1], (float)W, th[0])));
      tv[v] = t;
      if (t_hat) t_hat[v] = t;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int best = 0;
    for (int v = 1; v < kNumVariants; ++v)
      if (tv[v] < tv[best]) best = v;
    *variant = best;
  }
}

}  // namespace

hipError_t launch_select_config(const moe_problem& p, const int32_t* counts, const float* theta,
                                const CostTable& tab, int32_t* variant, float* t_hat,
                                hipStream_t s) {
  const int threads = kWave * (kNumVariants < 16 ? kNumVariants : 16);
  select_config_kernel<<<1, threads, 0, s>>>(counts, p.local_experts, theta, tab, variant, t_hat);
  return hipGetLastError();
}

}  // namespace moe
