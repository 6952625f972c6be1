// align_sort.hip -- step 3: group the routed slots by local expert and pad every
// group to the chosen configuration's tile rows.
//
// RaMP (arXiv 2604.26039) 3.2: the selection kernel writes the tokens grouped by
// expert and padded into the chosen configuration's tiles.  The pages give no
// layout; the one used here: experts in ascending local index, each expert's slots
// s = t*k + j in ascending s (a stable counting sort), padded with -1 to a multiple
// of b = BLOCK_M of the chosen configuration; an expert with no token gets no tile
// (ceil(0/b) = 0, as in Eq. 1).  Outputs: sorted_slots [R], block_expert[R/b],
// num_blocks, and the inverse map slot_pos (-1 for slots of other GPUs' experts).
//
// Design (one workgroup of 16 waves; the whole step stays in LDS):
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
namespace {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;

__device__ __forceinline__ void build_masks(unsigned long long* masks, const int32_t* ids, int blk,
                                            int B, int k, int e0, int E_loc, int lane) {
  for (int e = lane; e < E_loc; e += kWave) masks[e] = 0ull;
  __builtin_amdgcn_wave_barrier();
  const int t = blk * kWave + lane;
  if (t < B) {
    for (int j = 0; j < k; ++j) {
      const int e = ids[(int64_t)t * k + j] - e0;
      if (e >= 0 && e < E_loc) atomicOr(&masks[e], 1ull << lane);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

__global__ void __launch_bounds__(kAlignThreads)
align_sort_kernel(const int32_t* __restrict__ ids, const int32_t* __restrict__ variant, int B,
                  int k, int e0, int E_loc, int32_t* __restrict__ sorted_slots,
                  int32_t* __restrict__ block_expert, int32_t* __restrict__ num_blocks,
                  int32_t* __restrict__ slot_pos) {
  extern __shared__ unsigned long long lds_u64[];
  const int nblk = (B + kWave - 1) / kWave;
  unsigned long long* masks_all = lds_u64;                              // [16][E_loc]
  int32_t* base = (int32_t*)(lds_u64 + (size_t)kAlignWaves * E_loc);     // [nblk][E_loc]
  int32_t* off = base + (size_t)nblk * E_loc;                           // [E_loc + 1]
  int32_t* tot = off + E_loc + 1;                                       // [E_loc]
  __shared__ int wave_tot[kAlignWaves];
  __shared__ int s_b;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  unsigned long long* masks = masks_all + (size_t)wave * E_loc;

  if (tid == 0) {
    const int v = *variant;
    s_b = (v >= 0 && v < kNumVariants) ? kVariants[v].bm : 0;
  }
  __syncthreads();
  const int b = s_b;
  if (b == 0) {  // configuration index out of range: no tiles, no local slots
    for (int64_t s = tid; s < (int64_t)B * k; s += kAlignThreads) slot_pos[s] = -1;
    if (tid == 0) *num_blocks = 0;
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
  if (tid == 0) *num_blocks = nb;

  // pass 3: padding rows [off[e] + n_e, off[e + 1]) and the block -> expert table
  if (tid < E_loc)
    for (int r = off[tid] + tot[tid]; r < off[tid + 1]; ++r) sorted_slots[r] = -1;
  for (int i = tid; i < nb; i += kAlignThreads) {
    const int row = i * b;
    int lo = 0, hi = E_loc - 1;  // the largest e with off[e] <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= row) lo = mid; else hi = mid - 1;
    }
    block_expert[i] = lo;
  }
  __syncthreads();

  // pass 4: stable scatter
  for (int blk = wave; blk < nblk; blk += kAlignWaves) {
    build_masks(masks, ids, blk, B, k, e0, E_loc, lane);
    const int t = blk * kWave + lane;
    if (t < B) {
      const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
      for (int j = 0; j < k; ++j) {
        const int64_t s = (int64_t)t * k + j;
        const int e = ids[s] - e0;
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

}  // namespace

size_t align_lds_bytes(int B, int E_loc) {
  const size_t nblk = (size_t)(B + kWave - 1) / kWave;
  return (size_t)kAlignWaves * E_loc * 8 + nblk * E_loc * 4 + (size_t)(2 * E_loc + 1) * 4;
}

hipError_t launch_align_sort(const moe_problem& p, const int32_t* ids, const int32_t* variant,
                             int32_t* sorted_slots, int32_t* block_expert, int32_t* num_blocks,
                             int32_t* slot_pos, hipStream_t s) {
  const size_t lds = align_lds_bytes(p.tokens, p.local_experts);
  if (lds > 64 * 1024) {
    // opt in to more than 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU)
    static int done[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && !done[dev]) {
      if (hipFuncSetAttribute((const void*)align_sort_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess)
        done[dev] = 1;
      else
        (void)hipGetLastError();
    }
  }
  align_sort_kernel<<<1, kAlignThreads, lds, s>>>(ids, variant, p.tokens, p.top_k, p.expert_begin,
                                                  p.local_experts, sorted_slots, block_expert,
                                                  num_blocks, slot_pos);
  return hipGetLastError();
}

}  // namespace moe
