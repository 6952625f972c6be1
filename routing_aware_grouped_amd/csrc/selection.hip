// selection.hip -- steps 1 to 3 of the layer: top-k routing with the per-expert
// histogram, the on-GPU choice of the tile configuration, and the stable grouping
// of the routed slots into padded tiles; each as its own kernel (the three C entry
// points) and fused (moe_route_select_align): one workgroup for batches one
// workgroup routes, else the routing launch then one select+align launch.
//
// ---- step 1 ----
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
//
// ---- step 2 ----
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
//
// ---- step 3 ----
//
// RaMP (arXiv 2604.26039) 3.2: the selection kernel writes the tokens grouped by
// expert and padded into the chosen configuration's tiles.  The pages give no
// layout; the one used here: experts in ascending local index, each expert's slots
// s = t*k + j in ascending s (a stable counting sort), padded with -1 to a multiple
// of b = BLOCK_M of the chosen configuration; an expert with no token gets no tile
// (ceil(0/b) = 0, as in Eq. 1).  Outputs: sorted_slots [R], block_expert[R/b],
// num_blocks, and the inverse map slot_pos (-1 for slots of other GPUs' experts).
//
// Design (workgroups of 16 waves; the whole step stays in LDS; a grid of up to 64
// workgroups, one per 64-token block, where each repeats passes 1-2 and writes its
// share of passes 3-4):
//   * a token's k experts are distinct, so inside one expert ascending s means
//     ascending token t.  Tokens are cut into 64-token blocks, one lane per token.
//     For a block, each wave builds a 64-bit lane mask per expert in LDS (bit i set
//     when token blk*64+i is routed to that expert; LDS atomic OR).  The rank of a
//     token inside its expert within the block is popcount(mask & lanes-below).
//   * pass 1 stores popcount(mask) per (block, expert); pass 2 turns those into
//     each block's first row per expert (exclusive prefix over blocks, plus the
//     expert's padded offset from a scan over experts); pass 3 writes padding and
//     the block->expert table; pass 4 rebuilds the block masks and scatters.
// The permutation is therefore deterministic and equals the stable order exactly.
#include "moe_common.h"

namespace moe {

size_t align_lds_bytes(int B, int E_loc);

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

// Cross-lane reductions over groups of L lanes (L = 8, 16, 32 or 64) with DPP
// moves, which run in the vector ALU instead of the LDS crossbar that a generic
// shuffle goes through: quad swaps, the half-row and row mirrors (8 and 16 lanes),
// then for 32 and 64 lanes the row broadcasts of the scan pattern, after which the
// group's last lane holds the result and is read back with readlane.  Every lane of
// the wave must take part; every lane of a group gets the same value.  `id` is the
// operation's identity, which lanes outside the broadcast's row mask receive.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v, uint32_t id) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROWMASK, 0xF, false);
}

template <int L, class Op>
__device__ __forceinline__ uint32_t group_reduce(uint32_t v, uint32_t id, Op op) {
  static_assert(L == 8 || L == 16 || L == 32 || L == 64, "group of 8 to 64 lanes");
  v = op(v, dpp_mov<0xB1, 0xF>(v, id));   // quad_perm [1,0,3,2]
  v = op(v, dpp_mov<0x4E, 0xF>(v, id));   // quad_perm [2,3,0,1]
  v = op(v, dpp_mov<0x141, 0xF>(v, id));  // row_half_mirror: 8 lanes
  if (L >= 16) v = op(v, dpp_mov<0x140, 0xF>(v, id));  // row_mirror: 16 lanes
  if (L >= 32) v = op(v, dpp_mov<0x142, 0xA>(v, id));  // row_bcast:15 into rows 1, 3
  if (L == 64) {
    v = op(v, dpp_mov<0x143, 0xC>(v, id));  // row_bcast:31 into rows 2, 3
    v = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  } else if (L == 32) {
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
    v = (threadIdx.x & 32) ? b : a;
  }
  return v;
}

// The largest 64-bit key of the group: the largest high word, then among the lanes
// holding it the largest low word.
template <int L>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  auto umax = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  const uint32_t hi = group_reduce<L>((uint32_t)(v >> 32), 0u, umax);
  const uint32_t lo = group_reduce<L>((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u, 0u, umax);
  return ((uint64_t)hi << 32) | lo;
}

struct IAdd {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};

template <int L>
__device__ __forceinline__ float group_sum_f32(float v) {
  auto add = [](uint32_t a, uint32_t b) { return __float_as_uint(__uint_as_float(a) + __uint_as_float(b)); };
  return __uint_as_float(group_reduce<L>(__float_as_uint(v), 0u, add));
}

__global__ void zero_counts_kernel(int32_t* counts, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) counts[i] = 0;
}

// One workgroup's share of the routing: tokens wg * groups, (wg + nwg) * groups, ...
// NT threads, L lanes per token, MMAX >= ceil(E / L) logits per lane; hist [E_loc]
// in LDS collects this workgroup's local-expert counts.  With lds_ids (one
// workgroup for the whole batch) the ids also go to LDS, [B][k], for the alignment
// that follows.  Every logit load is unconditional (out-of-range lanes read
// element 0 of a valid row and discard it), so one wait covers them all.
template <int NT, int L, int MMAX>
__device__ __forceinline__ void route_block(const float* __restrict__ logits, int32_t* __restrict__ ids,
                                            float* __restrict__ wout, int32_t* hist, int B, int E,
                                            int k, int e0, int E_loc, int renormalize, int wg,
                                            int nwg, int32_t* lds_ids) {
  for (int i = threadIdx.x; i < E_loc; i += NT) hist[i] = 0;
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int gl = lane & (L - 1);  // lane inside the token group
  constexpr int groups_per_wg = NT / L;
  const int group = threadIdx.x / L;
  const int M = (E + L - 1) / L;

  for (int t0 = wg * groups_per_wg; t0 < B; t0 += nwg * groups_per_wg) {
    const int t = t0 + group;
    const bool active = t < B;  // whole groups are inactive together
    uint64_t key[MMAX];
    const float* lrow = logits + (int64_t)(active ? t : 0) * E;
    float xl[MMAX];
#pragma unroll
    for (int i = 0; i < MMAX; ++i) {
      const int e = gl + i * L;
      xl[i] = lrow[(i < M && e < E) ? e : 0];
    }
#pragma unroll
    for (int i = 0; i < MMAX; ++i) {
      const int e = gl + i * L;
      key[i] = (active && i < M && e < E)
                   ? ((uint64_t)float_order_key(xl[i]) << 32) | (uint32_t)(~(uint32_t)e)
                   : 0;
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
      float xr[MMAX];
#pragma unroll
      for (int i = 0; i < MMAX; ++i) {
        const int e = gl + i * L;
        xr[i] = lrow[(i < M && e < E) ? e : 0];
      }
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < MMAX; ++i) {
        const int e = gl + i * L;
        if (active && i < M && e < E) part += expf(xr[i] - top);
      }
      den = group_sum_f32<L>(part);
    }
    if (active && gl < k) {
      ids[(int64_t)t * k + gl] = my_id;
      if (lds_ids) lds_ids[t * k + gl] = my_id;
      wout[(int64_t)t * k + gl] = ex / den;
      const int le = my_id - e0;
      if (le >= 0 && le < E_loc) atomicAdd(&hist[le], 1);
    }
  }
  __syncthreads();
}

template <int NT, int L, int MMAX>
__global__ void __launch_bounds__(NT) route_topk_kernel(const float* __restrict__ logits, int32_t* __restrict__ ids,
                                  float* __restrict__ wout, int32_t* __restrict__ counts, int B,
                                  int E, int k, int e0, int E_loc, int renormalize,
                                  int single_wg) {
  extern __shared__ int32_t hist[];  // [E_loc]
  route_block<NT, L, MMAX>(logits, ids, wout, hist, B, E, k, e0, E_loc, renormalize, blockIdx.x,
                           gridDim.x, nullptr);
  if (single_wg) {
    for (int i = threadIdx.x; i < E_loc; i += NT) counts[i] = hist[i];
  } else {
    for (int i = threadIdx.x; i < E_loc; i += NT)
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
    // at most two workgroups per CU: each then routes several token groups and
    // adds its LDS histogram to the counts once, which cuts the global atomics
    if (grid > 512) grid = 512;
    zero_counts_kernel<<<(p.local_experts + 255) / 256, 256, 0, s>>>(counts, p.local_experts);
  }
  if (single)
    route_topk_kernel<1024, L, MMAX><<<grid, threads, p.local_experts * sizeof(int32_t), s>>>(
        logits, ids, w, counts, B, p.num_experts, p.top_k, p.expert_begin, p.local_experts,
        p.renormalize, 1);
  else
    route_topk_kernel<256, L, MMAX><<<grid, threads, p.local_experts * sizeof(int32_t), s>>>(
        logits, ids, w, counts, B, p.num_experts, p.top_k, p.expert_begin, p.local_experts,
        p.renormalize, 0);
  return hipGetLastError();
}



// The selection by one workgroup of NT threads (one wave per configuration):
// counts may be in global memory or LDS.  Returns the chosen index to every thread.
template <int NT>
__device__ __forceinline__ int select_block(const int32_t* counts, int E_loc,
                                            const float* __restrict__ theta, const CostTable& tab,
                                            int32_t* __restrict__ variant,
                                            float* __restrict__ t_hat) {
  __shared__ float tv[kNumVariants];
  __shared__ int active;
  __shared__ int chosen;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  constexpr int nwaves = NT / kWave;
  if (threadIdx.x == 0) active = 0;
  __syncthreads();
  if (wave == 0) {
    int a = 0;
    for (int e = lane; e < E_loc; e += kWave) a += counts[e] > 0;
    a = (int)group_reduce<kWave>((uint32_t)a, 0u, IAdd{});
    if (lane == 0) active = a;
  }
  __syncthreads();
  for (int v = wave; v < kNumVariants; v += nwaves) {
    const int b = tab.b[v];
    int rt = 0;
    for (int e = lane; e < E_loc; e += kWave) rt += (counts[e] + b - 1) / b;
    rt = (int)group_reduce<kWave>((uint32_t)rt, 0u, IAdd{}) + tab.rt_shared[v];
    if (lane == 0) {
      const int T1 = tab.q1[v] * rt, T2 = tab.q2[v] * rt;
      const int W = (T1 + tab.S1[v] - 1) / tab.S1[v] + (T2 + tab.S2[v] - 1) / tab.S2[v];
      const int T = T1 + T2;
      const float* th = theta + 4 * v;
      const float t = __builtin_fmaf(
          th[3], (float)(active + tab.a_shared),
          __builtin_fmaf(th[2], (float)T, __builtin_fmaf(th[1], (float)W, th[0])));
      tv[v] = t;
      if (t_hat && blockIdx.x == 0) t_hat[v] = t;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int best = 0;
    for (int v = 1; v < kNumVariants; ++v)
      if (tv[v] < tv[best]) best = v;
    if (blockIdx.x == 0) *variant = best;  // every workgroup of a grid chooses the same
    chosen = best;
  }
  __syncthreads();
  return chosen;
}

__global__ void select_config_kernel(const int32_t* __restrict__ counts, int E_loc,
                                     const float* __restrict__ theta, CostTable tab,
                                     int32_t* __restrict__ variant, float* __restrict__ t_hat) {
  select_block<kWave * (kNumVariants < 16 ? kNumVariants : 16)>(counts, E_loc, theta, tab, variant,
                                                              t_hat);
}



constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;

// Bytes of LDS the alignment's tables take: 16 waves' expert masks, the per-block
// bases [nblk][E_loc], the expert offsets [E_loc + 1] and totals [E_loc].
__host__ __device__ __forceinline__ size_t align_table_bytes(int B, int E_loc) {
  const size_t nblk = (size_t)(B + kWave - 1) / kWave;
  return (size_t)kAlignWaves * E_loc * 8 + nblk * E_loc * 4 + (size_t)(2 * E_loc + 1) * 4;
}

// Local expert index of a routed id: ids are global expert ids (int32_t), or local
// indices staged in LDS as bytes with 255 for an expert of another GPU (uint8_t).
__device__ __forceinline__ int local_of(int32_t v, int e0) { return v - e0; }
__device__ __forceinline__ int local_of(uint8_t v, int) { return v == 255 ? -1 : (int)v; }

template <typename IdT>
__device__ __forceinline__ void build_masks(unsigned long long* masks, const IdT* ids, int blk,
                                            int B, int k, int e0, int E_loc, int lane) {
  for (int e = lane; e < E_loc; e += kWave) masks[e] = 0ull;
  __builtin_amdgcn_wave_barrier();
  const int t = blk * kWave + lane;
  const int tc = t < B ? t : B - 1;  // loads stay in bounds; results of t >= B are dropped
  for (int j0 = 0; j0 < k; j0 += 4) {
    IdT v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = ids[(int64_t)tc * k + (j0 + u < k ? j0 + u : k - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = local_of(v[u], e0);
      if (t < B && j0 + u < k && e >= 0 && e < E_loc) atomicOr(&masks[e], 1ull << lane);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// The alignment for tile rows b (b = 0: no valid configuration, so no tiles and no
// local slots) by a grid of workgroups of kAlignThreads threads; lds_u64 holds
// align_lds_bytes(B, E_loc) bytes.  Every workgroup computes the counts and the
// offsets (passes 1-2) in full; the writes (passes 3-4) are divided among the
// workgroups: padding rows by expert, block_expert by row-block and the scatter
// by 64-token block.  The scatter is bound by one CU's store path (64 scattered
// 4-byte stores per wave instruction), which the division spreads over CUs.
template <typename IdT>
__device__ __forceinline__ void align_block(const IdT* __restrict__ ids, int b, int B, int k,
                                            int e0, int E_loc, int32_t* __restrict__ sorted_slots,
                                            int32_t* __restrict__ block_expert,
                                            int32_t* __restrict__ num_blocks,
                                            int32_t* __restrict__ slot_pos,
                                            unsigned long long* lds_u64) {
  const int nblk = (B + kWave - 1) / kWave;
  unsigned long long* masks_all = lds_u64;                              // [16][E_loc]
  int32_t* base = (int32_t*)(lds_u64 + (size_t)kAlignWaves * E_loc);     // [nblk][E_loc]
  int32_t* off = base + (size_t)nblk * E_loc;                           // [E_loc + 1]
  int32_t* tot = off + E_loc + 1;                                       // [E_loc]
  __shared__ int wave_tot[kAlignWaves];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  unsigned long long* masks = masks_all + (size_t)wave * E_loc;

  const int wg = blockIdx.x, nwg = gridDim.x;
  if (b == 0) {  // configuration index out of range: no tiles, no local slots
    for (int64_t s = (int64_t)wg * kAlignThreads + tid; s < (int64_t)B * k;
         s += (int64_t)nwg * kAlignThreads)
      slot_pos[s] = -1;
    if (wg == 0 && tid == 0) *num_blocks = 0;
    return;
  }

  // pass 1: per-(block, expert) counts
  for (int blk = wave; blk < nblk; blk += kAlignWaves) {
    build_masks(masks, ids, blk, B, k, e0, E_loc, lane);
    for (int e = lane; e < E_loc; e += kWave)
      base[(size_t)blk * E_loc + e] = __popcll(masks[e]);
  }
  __syncthreads();

  // pass 2: per expert (one thread each, E_loc <= 1024): exclusive prefix over
  // blocks, the padded size, then an exclusive scan of padded sizes over experts
  {
    const int e = tid;
    int padded = 0;
    if (e < E_loc) {
      int run = 0;
      for (int blk = 0; blk < nblk; ++blk) {
        const int c = base[(size_t)blk * E_loc + e];
        base[(size_t)blk * E_loc + e] = run;
        run += c;
      }
      tot[e] = run;
      padded = (run + b - 1) / b * b;
    }
    int incl = padded;  // wave-inclusive scan
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
      int wt = lane < kAlignWaves ? wave_tot[lane] : 0;
      for (int d = 1; d < kAlignWaves; d <<= 1) {
        const int o = __shfl_up(wt, d, kWave);
        if (lane >= d) wt += o;
      }
      if (lane < kAlignWaves) wave_tot[lane] = wt;  // inclusive over waves
    }
    __syncthreads();
    const int before = (wave == 0 ? 0 : wave_tot[wave - 1]) + incl - padded;
    if (e < E_loc) off[e] = before;
    if (e == E_loc - 1) off[E_loc] = before + padded;
  }
  __syncthreads();
  for (int i = tid; i < nblk * E_loc; i += kAlignThreads) base[i] += off[i % E_loc];
  const int R = off[E_loc];
  const int nb = R / b;
  if (wg == 0 && tid == 0) *num_blocks = nb;

  // pass 3: padding rows [off[e] + n_e, off[e + 1]), one wave per expert, and the
  // block -> expert table
  for (int e = wg * kAlignWaves + wave; e < E_loc; e += nwg * kAlignWaves)
    for (int r = off[e] + tot[e] + lane; r < off[e + 1]; r += kWave) sorted_slots[r] = -1;
  for (int i = wg * kAlignThreads + tid; i < nb; i += nwg * kAlignThreads) {
    const int row = i * b;
    int lo = 0, hi = E_loc - 1;  // the largest e with off[e] <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= row) lo = mid; else hi = mid - 1;
    }
    block_expert[i] = lo;
  }
  __syncthreads();

  // pass 4: stable scatter; workgroup wg takes blocks wg, wg + nwg, ...
  for (int blk = wave * nwg + wg; blk < nblk; blk += kAlignWaves * nwg) {
    build_masks(masks, ids, blk, B, k, e0, E_loc, lane);
    const int t = blk * kWave + lane;
    const int tc = t < B ? t : B - 1;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    for (int j0 = 0; j0 < k; j0 += 4) {
      IdT v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = ids[(int64_t)tc * k + (j0 + u < k ? j0 + u : k - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (t >= B || j0 + u >= k) continue;
        const int64_t s = (int64_t)t * k + j0 + u;
        const int e = local_of(v[u], e0);
        if (e >= 0 && e < E_loc) {
          const int pos = base[(size_t)blk * E_loc + e] + __popcll(masks[e] & below);
          sorted_slots[pos] = (int32_t)s;
          slot_pos[s] = pos;
        } else {
          slot_pos[s] = -1;
        }
      }
    }
  }
}

// Workgroups of an alignment grid: one per 64-token block, at most kAlignMaxWg.
constexpr int kAlignMaxWg = 64;
inline int align_grid(int B) {
  const int nblk = (B + kWave - 1) / kWave;
  return nblk < 1 ? 1 : (nblk < kAlignMaxWg ? nblk : kAlignMaxWg);
}

__device__ __forceinline__ int tile_rows(int v) {
  return (v >= 0 && v < kNumVariants) ? kVariants[v].bm : 0;
}

__global__ void __launch_bounds__(kAlignThreads)
align_sort_kernel(const int32_t* __restrict__ ids, const int32_t* __restrict__ variant, int B,
                  int k, int e0, int E_loc, int32_t* __restrict__ sorted_slots,
                  int32_t* __restrict__ block_expert, int32_t* __restrict__ num_blocks,
                  int32_t* __restrict__ slot_pos) {
  extern __shared__ unsigned long long lds_u64[];
  __shared__ int s_b;
  if (threadIdx.x == 0) s_b = tile_rows(*variant);
  __syncthreads();
  align_block(ids, s_b, B, k, e0, E_loc, sorted_slots, block_expert, num_blocks, slot_pos, lds_u64);
}


// ---- fused steps 1-3 ----

// The configuration in *variant, to every thread (theta == NULL: no selection).
__device__ __forceinline__ int given_variant(const int32_t* variant) {
  __shared__ int sv;
  if (threadIdx.x == 0) sv = *variant;
  __syncthreads();
  return sv;
}

// Steps 1-3 in one workgroup of 1024 threads, for a batch one workgroup routes:
// the routing with the histogram in LDS, the counts, the choice from the LDS
// counts (or the given configuration), then the alignment for the chosen tile
// rows.  The alignment reads the ids this workgroup wrote; the barriers in
// between order those accesses.
template <int L, int MMAX>
__global__ void __launch_bounds__(1024)
route_select_align_kernel(const float* __restrict__ logits, const float* __restrict__ theta,
                          CostTable tab, int32_t* __restrict__ ids, float* __restrict__ wout,
                          int32_t* __restrict__ counts, int32_t* __restrict__ variant,
                          float* __restrict__ t_hat, int32_t* __restrict__ sorted_slots,
                          int32_t* __restrict__ block_expert, int32_t* __restrict__ num_blocks,
                          int32_t* __restrict__ slot_pos, int B, int E, int k, int e0, int E_loc,
                          int renormalize) {
  extern __shared__ unsigned long long lds_u64[];
  __shared__ float th_s[4 * kNumVariants];
  // LDS: hist [E_loc], the alignment's tables, then the ids [B][k]
  int32_t* hist = (int32_t*)lds_u64;
  unsigned long long* al = lds_u64 + (E_loc + 1) / 2;
  int32_t* lds_ids = (int32_t*)((char*)al + align_table_bytes(B, E_loc));
  // the cost-model coefficients are loaded before the routing and kept in flight
  const bool pre = theta != nullptr && threadIdx.x < 4 * kNumVariants;
  const float th = pre ? theta[threadIdx.x] : 0.f;
  route_block<1024, L, MMAX>(logits, ids, wout, hist, B, E, k, e0, E_loc, renormalize, 0, 1,
                             lds_ids);
  if (pre) th_s[threadIdx.x] = th;  // read after select_block's first barrier
  for (int i = threadIdx.x; i < E_loc; i += 1024) counts[i] = hist[i];
  const int v = theta ? select_block<1024>(hist, E_loc, th_s, tab, variant, t_hat) : given_variant(variant);
  align_block(lds_ids, tile_rows(v), B, k, e0, E_loc, sorted_slots, block_expert, num_blocks,
              slot_pos, al);
}

// Steps 2-3 after a multi-workgroup routing launch, on the alignment grid (every
// workgroup makes the same choice; workgroup 0 writes it).  With
// stage_ids the ids are first copied into LDS after the alignment's tables (16-byte
// loads, issued before the selection so that they overlap it), and both alignment
// passes read them there: stage_ids 1 copies the int32 ids, 2 stores each as its
// local expert index in one byte (255: another GPU's expert; needs E_loc < 255),
// for batches whose int32 ids would not fit.
__global__ void __launch_bounds__(kAlignThreads)
select_align_kernel(const int32_t* __restrict__ counts, const float* __restrict__ theta,
                    CostTable tab, const int32_t* __restrict__ ids, int32_t* __restrict__ variant,
                    float* __restrict__ t_hat, int32_t* __restrict__ sorted_slots,
                    int32_t* __restrict__ block_expert, int32_t* __restrict__ num_blocks,
                    int32_t* __restrict__ slot_pos, int B, int k, int e0, int E_loc,
                    int stage_ids) {
  extern __shared__ unsigned long long lds_u64[];
  // after the tables, at a 16-byte boundary
  int32_t* lds_ids = (int32_t*)((char*)lds_u64 + (align_table_bytes(B, E_loc) + 15) / 16 * 16);
  uint8_t* lds_loc = (uint8_t*)lds_ids;
  const int n = B * k;
  const int n4 = n / 4;  // ids is 16-byte aligned (checked by the host before staging)
  if (stage_ids == 1) {
    for (int i = threadIdx.x; i < n4; i += kAlignThreads)
      ((u32x4*)lds_ids)[i] = ((const u32x4*)ids)[i];
    for (int i = n4 * 4 + threadIdx.x; i < n; i += kAlignThreads) lds_ids[i] = ids[i];
  } else if (stage_ids == 2) {
    auto loc = [&](int32_t id) __attribute__((always_inline)) {
      const int e = id - e0;
      return (uint32_t)(e >= 0 && e < E_loc ? e : 255);
    };
    for (int i = threadIdx.x; i < n4; i += kAlignThreads) {
      const u32x4 q = ((const u32x4*)ids)[i];
      ((uint32_t*)lds_loc)[i] = loc((int32_t)q[0]) | loc((int32_t)q[1]) << 8 |
                                loc((int32_t)q[2]) << 16 | loc((int32_t)q[3]) << 24;
    }
    for (int i = n4 * 4 + threadIdx.x; i < n; i += kAlignThreads) lds_loc[i] = (uint8_t)loc(ids[i]);
  }
  // both paths below start with a barrier, which publishes the copy
  const int v = theta ? select_block<kAlignThreads>(counts, E_loc, theta, tab, variant, t_hat)
                      : given_variant(variant);
  if (stage_ids == 2)
    align_block(lds_loc, tile_rows(v), B, k, e0, E_loc, sorted_slots, block_expert, num_blocks,
                slot_pos, lds_u64);
  else
    align_block(stage_ids ? lds_ids : ids, tile_rows(v), B, k, e0, E_loc, sorted_slots,
                block_expert, num_blocks, slot_pos, lds_u64);
}

// more than 64 KiB of dynamic LDS needs an opt-in (gfx950 has 160 KiB per CU); the
// attribute is raised only when a launch needs more than any earlier one did
hipError_t allow_lds(const void* fn, size_t bytes) { return opt_in_lds(fn, (int)bytes); }

template <int L, int MMAX>
hipError_t launch_rsa(const moe_problem& p, const float* logits, const float* theta,
                      const CostTable& tab, int32_t* ids, float* w, int32_t* counts,
                      int32_t* variant, float* t_hat, int32_t* sorted_slots,
                      int32_t* block_expert, int32_t* num_blocks, int32_t* slot_pos,
                      hipStream_t s) {
  const int B = p.tokens;
  const size_t al_bytes = align_lds_bytes(B, p.local_experts);
  const size_t fused_bytes =
      (size_t)(p.local_experts + 1) / 2 * 8 + al_bytes + (size_t)B * p.top_k * sizeof(int32_t);
  if (B <= 4 * (1024 / L) && fused_bytes <= 150 * 1024) {
    const void* fn = (const void*)route_select_align_kernel<L, MMAX>;
    hipError_t e = allow_lds(fn, fused_bytes);
    if (e != hipSuccess) return e;
    route_select_align_kernel<L, MMAX><<<1, 1024, fused_bytes, s>>>(
        logits, theta, tab, ids, w, counts, variant, t_hat, sorted_slots, block_expert,
        num_blocks, slot_pos, B, p.num_experts, p.top_k, p.expert_begin, p.local_experts,
        p.renormalize);
    return hipGetLastError();
  }
  hipError_t e = launch_lm<L, MMAX>(p, logits, ids, w, counts, s);
  if (e != hipSuccess) return e;
  // the ids go to LDS too when they fit beside the tables (and are 16-byte aligned)
  const size_t ids_bytes = (size_t)B * p.top_k * sizeof(int32_t);
  const size_t al16 = (al_bytes + 15) / 16 * 16;
  const size_t loc_bytes = ((size_t)B * p.top_k + 15) / 16 * 16;
  const bool aligned16 = ((uintptr_t)ids & 15) == 0;
  int stage = 0;
  if (aligned16 && al16 + ids_bytes <= 150 * 1024)
    stage = 1;
  else if (aligned16 && p.local_experts < 255 && al16 + loc_bytes <= 150 * 1024)
    stage = 2;
  const size_t lds = stage == 1 ? al16 + ids_bytes : (stage == 2 ? al16 + loc_bytes : al_bytes);
  e = allow_lds((const void*)select_align_kernel, lds);
  if (e != hipSuccess) return e;
  select_align_kernel<<<align_grid(B), kAlignThreads, lds, s>>>(
      counts, theta, tab, ids, variant, t_hat, sorted_slots, block_expert, num_blocks, slot_pos, B,
      p.top_k, p.expert_begin, p.local_experts, stage);
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


hipError_t launch_select_config(const moe_problem& p, const int32_t* counts, const float* theta,
                                const CostTable& tab, int32_t* variant, float* t_hat,
                                hipStream_t s) {
  const int threads = kWave * (kNumVariants < 16 ? kNumVariants : 16);
  select_config_kernel<<<1, threads, 0, s>>>(counts, p.local_experts, theta, tab, variant, t_hat);
  return hipGetLastError();
}


size_t align_lds_bytes(int B, int E_loc) { return align_table_bytes(B, E_loc); }

hipError_t launch_align_sort(const moe_problem& p, const int32_t* ids, const int32_t* variant,
                             int32_t* sorted_slots, int32_t* block_expert, int32_t* num_blocks,
                             int32_t* slot_pos, hipStream_t s) {
  const size_t lds = align_lds_bytes(p.tokens, p.local_experts);
  hipError_t e = allow_lds((const void*)align_sort_kernel, lds);
  if (e != hipSuccess) return e;
  align_sort_kernel<<<align_grid(p.tokens), kAlignThreads, lds, s>>>(
      ids, variant, p.tokens, p.top_k, p.expert_begin, p.local_experts, sorted_slots, block_expert,
      num_blocks, slot_pos);
  return hipGetLastError();
}


hipError_t launch_route_select_align(const moe_problem& p, const float* logits,
                                     const float* theta, const CostTable& tab, int32_t* ids,
                                     float* w, int32_t* counts, int32_t* variant, float* t_hat,
                                     int32_t* sorted_slots, int32_t* block_expert,
                                     int32_t* num_blocks, int32_t* slot_pos, hipStream_t s) {
#define MOE_RSA(L, M) \
  launch_rsa<L, M>(p, logits, theta, tab, ids, w, counts, variant, t_hat, sorted_slots, \
                   block_expert, num_blocks, slot_pos, s)
  const int E = p.num_experts;
  if (E <= 8) return MOE_RSA(8, 1);
  if (E <= 16) return MOE_RSA(16, 1);
  if (E <= 32) return MOE_RSA(32, 1);
  if (E <= 64) return MOE_RSA(64, 1);
  if (E <= 128) return MOE_RSA(64, 2);
  if (E <= 256) return MOE_RSA(64, 4);
  if (E <= 512) return MOE_RSA(64, 8);
  if (E <= 1024) return MOE_RSA(64, 16);
  return MOE_RSA(64, 64);
#undef MOE_RSA
}

}  // namespace moe
