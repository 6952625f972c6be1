// fused_ffn.hip -- the fused plan for small batches: gate/up, SwiGLU and a slice of
// the down projection in one launch, then a combine that adds the slices.
//
// RaMP (arXiv 2604.26039) appendix A.8, "Fusion": a tile runs the up-projection,
// the gated activation and the down-projection in turn, and adds its down-
// projection result into the layer's output.  Here a tile is one row-block of the
// alignment (up to BLOCK_M token rows of one expert e, BLOCK_M of the chosen
// configuration) times one slice of kSlice columns of the intermediate size I:
//   g, u = X W1_e[slice]^T, X W3_e[slice]^T     (reduction over H, fp32)
//   h    = bf16(silu(g) u)                      (the intermediate precision; LDS)
//   y_j  = h W2_e[:, slice]^T                   (reduction over the slice, fp32)
// The slices of one slot are not added with atomics, whose order would depend on
// timing: tile j writes its fp32 rows y_j to part[j][slot][:] (slot = t k + i, the
// routed slot id), and the combine adds a slot's I / kSlice slices in a fixed
// order, then the slots with their router weights.  Nothing has to be zeroed
// first and no workgroup waits for another.
//
// Cost: each tile streams its slice of W1, W3 and W2 once, and the FFN is one
// launch where the grouped plan enqueues four.  The partial rows add
// slots * H * 4 bytes per slice, written once and read once: small while a row-
// block holds a few token rows, which is where launches, not bytes, set the
// layer's time.  The caller picks the plan by batch size.
//
// Design (gfx950).  256 threads, four waves, no LDS staging of operands:
//   - gate/up: wave w takes one matrix (w & 1: W1 or W3) and half of the slice's
//     columns (w >> 1): one 16-column MFMA fragment, over the whole reduction,
//     on two 16-row groups of the pass's 32 token rows (v_mfma_f32_16x16x32_bf16).
//     Fragments go from memory straight into registers (buffer loads, 16 bytes
//     per lane), eight 32-deep steps per batch, the next batch in flight while
//     the current one is multiplied.  A step past the reduction's end loads with
//     an out-of-range offset, which returns zeros and reads no memory, so the loop
//     has no branch around its loads.
//   - fp8 weights are decoded in registers, w = q * s rounded to bf16, as the
//     grouped plan decodes them in staging (one scale per step: a 32-deep step of
//     16 rows lies in one 128 x 128 scale block).
//   - g and u meet in LDS as fp32, where h is formed in bf16.
//   - down: wave w takes every fourth 16-column group of H; a group is one
//     product over the 32-deep slice, with h's fragments read from LDS once per
//     pass and W2's loaded eight groups per batch, two batches in flight; the
//     first batch is issued before h is formed.
//   - two to four workgroups share a CU (the grid holds up to four per CU, so
//     every tile of a small batch is in flight at once).
//   - a row-block with more than 32 rows takes several passes over its slice.
#include <type_traits>

#include "fused_ffn.h"

namespace moe {
namespace {

constexpr int kSlice = 32;          // columns of I per tile
constexpr int kFusedThreads = 256;  // four waves
constexpr int kPassRows = 32;       // token rows per pass: two 16-row MFMA groups
constexpr int kStepBatch = 8;       // 32-deep gate/up steps per load batch (256 deep)
constexpr int kGroupBatch = 8;      // down-phase 16-column groups per load batch
constexpr uint32_t kNoOperand = 0x80000000u;  // past every operand buffer's range
constexpr int kStreamLoad = 2;      // cache policy of a buffer load: non-temporal
constexpr int kPkBlock = 256 * 64;  // bytes of one block of the packed weight copy

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

struct FusedArgs {
  const void* x;    // [B][H] bf16
  const void* w1;   // [E_loc][I][H] bf16 or fp8
  const void* w3;   // [E_loc][I][H]
  const void* w2;   // [E_loc][H][I]
  const float* s1;  // fp8 block scales: [E_loc][I/128][H/128] (s2: [E_loc][H/128][I/128])
  const float* s3;
  const float* s2;
  const int32_t* sorted_slots;
  const int32_t* block_expert;
  const int32_t* num_blocks;
  const int32_t* variant;
  float* part;      // [I / kSlice][slots][H]
  int32_t* status;  // the device status word (MOE_DEV_*)
  const uint8_t* wpk;  // the packed bf16 weight copy (moe_pack_wide), or null
  int H, I, k, E_loc, slots;
  int64_t rows_max;
};

// A weight fragment: 8 consecutive reduction values of one weight row.
template <bool FP8>
struct WFrag {
  u32x4 v;  // 8 bf16
};
template <>
struct WFrag<true> {
  u32x2 v;  // 8 E4M3FN codes
};

template <bool FP8>
__device__ __forceinline__ WFrag<FP8> load_w(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  WFrag<FP8> f;
  if constexpr (FP8)
    f.v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStreamLoad));
  else
    f.v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamLoad));
  return f;
}

template <bool FP8>
__device__ __forceinline__ bf16x8 decode(const WFrag<FP8>& f, float s) {
  if constexpr (FP8) {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(f.v[w], false);
      const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(f.v[w], true);
      o[2 * w] = bf16_pair(a[0] * s, a[1] * s);
      o[2 * w + 1] = bf16_pair(b[0] * s, b[1] * s);
    }
    return __builtin_bit_cast(bf16x8, o);
  } else {
    return __builtin_bit_cast(bf16x8, f.v);
  }
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu_times(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// one gate/up load batch of a wave: kStepBatch 32-deep steps, two token-row
// groups (A), one weight fragment (B) and its block scale (fp8) per step
template <bool FP8, int NG>
struct UpBatch {
  u32x4 a[kStepBatch][NG];
  WFrag<FP8> b[kStepBatch];
  float s[kStepBatch];
};

// one down-phase load batch of a wave: kGroupBatch column groups, one 32-deep W2
// fragment each, and each group's scale
template <bool FP8>
struct DownBatch {
  WFrag<FP8> b[kGroupBatch];
  float s[kGroupBatch];
};

template <bool FP8>
__global__ void __launch_bounds__(kFusedThreads, 2) fused_ffn_kernel(FusedArgs g) {
  __shared__ int s_slot[kPassRows];                              // slot id per pass row, -1: none
  __shared__ float s_gu[2][kPassRows][kSlice + 1];               // fp32 g (0) and u (1)
  __shared__ __attribute__((aligned(16))) uint16_t s_h[kPassRows][kSlice + 8];  // bf16 h rows

  // the device values the host cannot check: the chosen configuration and the
  // row-block count (workgroup 0 reports them)
  const int v = *g.variant;
  int nb = *g.num_blocks;
  int st = MOE_DEV_OK;
  int bm = 0;
  if (v < 0 || v >= kNumVariants) {
    st = MOE_DEV_BAD_VARIANT;
  } else {
    bm = kVariants[v].bm;
    const int64_t fit = g.rows_max / bm;
    if (nb < 0 || nb > fit) {
      st = MOE_DEV_BAD_BLOCKS;
      nb = nb < 0 ? 0 : (int)fit;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *g.status = st;
  if (st == MOE_DEV_BAD_VARIANT) return;

  constexpr int WSZ = FP8 ? 1 : 2;
  // the wave index through readfirstlane: values derived from it (the weight
  // matrix, the descriptors) are then known to be wave-uniform and live in scalar
  // registers; otherwise each buffer load becomes a loop over distinct descriptors
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int mt = wv & 1, half = wv >> 1;
  const int H = g.H, I = g.I;
  const int nsl = I / kSlice;
  const int nst = H / 32;                  // 32-deep gate/up steps
  const int nbt = (nst + kStepBatch - 1) / kStepBatch;  // gate/up load batches
  const int ncg = H / 64;                  // down-phase column groups per wave
  const int nbd = (ncg + kGroupBatch - 1) / kGroupBatch;  // down-phase load batches
  const __amdgpu_buffer_rsrc_t xr = buffer_of(g.x, (uint32_t)((int64_t)g.slots / g.k * H * 2));
  const int64_t tiles = (int64_t)nb * nsl;
  // the packed copy (bf16 only): blocks per expert and column tile, and where the
  // down blocks begin
  const bool pk = !FP8 && g.wpk != nullptr;
  const int nst1 = H / 32, ncol1 = (I + 127) / 128, nst2 = I / 32, ncol2 = (H + 255) / 256;
  const int64_t pk_gu = (int64_t)g.E_loc * ncol1 * nst1 * kPkBlock;

  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int j = (int)(t / nb), rb = (int)(t - (int64_t)j * nb);
    const int e = g.block_expert[rb];
    if (e < 0 || e >= g.E_loc) continue;  // the same value in every thread
    // this wave's 16 rows of its gate/up matrix, and expert e's W2: row-major, or
    // in the packed copy, whose 16 KiB blocks hold 256 rows x 32 reduction values
    // (gate/up: column tile n0 / 128 of 128 W1 rows then 128 W3 rows, one block per
    // 32-deep step; down: 256 W2 rows of one 32-deep slice of I, one block per
    // 256-row tile), so a wave's fragment load reads 1 KiB of consecutive bytes
    const int n0 = j * kSlice + half * 16;
    __amdgpu_buffer_rsrc_t wr, w2r;
    uint32_t boff;
    int sstep;  // buffer offset step per 32-deep gate/up step
    if (pk) {
      const int64_t blk = ((int64_t)e * ncol1 + n0 / 128) * nst1;
      wr = buffer_of(g.wpk + blk * kPkBlock, (uint32_t)(nst1 * kPkBlock));
      boff = (uint32_t)((mt * 128 + n0 % 128 + lr) * 64 + 16 * lg);
      sstep = kPkBlock;
      w2r = buffer_of(g.wpk + pk_gu + (int64_t)e * ncol2 * nst2 * kPkBlock,
                      (uint32_t)((int64_t)ncol2 * nst2 * kPkBlock));
    } else {
      wr = buffer_of((const char*)(mt ? g.w3 : g.w1) + ((int64_t)e * I + n0) * H * WSZ,
                     (uint32_t)(16 * H * WSZ));
      boff = (uint32_t)((lr * H + 8 * lg) * WSZ);
      sstep = 32 * WSZ;
      w2r = buffer_of((const char*)g.w2 + (int64_t)e * H * I * WSZ, (uint32_t)((int64_t)H * I * WSZ));
    }
    const float* sm = mt ? g.s3 : g.s1;
    const int64_t su0 = ((int64_t)e * (I / 128) + n0 / 128) * (H / 128);  // + 128-deep block
    const int64_t sd0 = (int64_t)e * (H / 128) * (I / 128) + (j * kSlice) / 128;  // + (n / 128) (I / 128)

    for (int r0 = 0; r0 < bm; r0 += kPassRows) {
      __syncthreads();  // the previous pass's readers of s_slot and s_h are done
      if (threadIdx.x < kPassRows) {
        int s = -1;
        if (r0 + (int)threadIdx.x < bm) s = g.sorted_slots[(int64_t)rb * bm + r0 + threadIdx.x];
        s_slot[threadIdx.x] = (s >= 0 && s < g.slots) ? s : -1;
      }
      __syncthreads();
      // the rows of a row-block that hold a slot come first
      if (s_slot[0] < 0) break;

      // one instance per row-group count: a pass whose rows 16..31 hold no slot
      // (the usual case at small batches) loads and multiplies one 16-row group
      auto pass = [&](auto ngc) __attribute__((always_inline)) {
        constexpr int NG = decltype(ngc)::value;
        // ---- gate/up over H ----
        uint32_t aoff[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          const int s = s_slot[gi * 16 + lr];
          aoff[gi] = s >= 0 ? (uint32_t)(((int64_t)(s / g.k) * H + 8 * lg) * 2) : kNoOperand;
        }

        auto load_up = [&](UpBatch<FP8, NG>& U, int bt) __attribute__((always_inline)) {
#pragma unroll
          for (int q = 0; q < kStepBatch; ++q) {
            const int st = bt * kStepBatch + q;
            const bool in = st < nst;
            const int k0 = st * 32;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
              U.a[q][gi] = __builtin_bit_cast(
                  u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, in ? aoff[gi] : kNoOperand, k0 * 2, 0));
            U.b[q] = load_w<FP8>(wr, in ? boff : kNoOperand, st * sstep);
            if constexpr (FP8) U.s[q] = sm[su0 + (in ? st / 4 : 0)];
          }
        };
        f32x4 acc[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) acc[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto mul_up = [&](const UpBatch<FP8, NG>& U) __attribute__((always_inline)) {
#pragma unroll
          for (int q = 0; q < kStepBatch; ++q) {
            const bf16x8 b = decode<FP8>(U.b[q], FP8 ? U.s[q] : 1.0f);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) acc[gi] = mfma(__builtin_bit_cast(bf16x8, U.a[q][gi]), b, acc[gi]);
          }
        };
        {
          UpBatch<FP8, NG> U0, U1;
          load_up(U0, 0);
          // steps past nst read zeros (an odd nbt runs one batch of zeros)
          for (int bt = 0; bt < nbt; bt += 2) {
            load_up(U1, bt + 1);
            mul_up(U0);
            load_up(U0, bt + 2);
            mul_up(U1);
          }
        }
        // the first W2 batch does not depend on h: its loads fly while h is formed
        const uint32_t doff0 = (uint32_t)((lr * (int64_t)I + j * kSlice + 8 * lg) * WSZ);
        auto load_down = [&](DownBatch<FP8>& D, int bd) __attribute__((always_inline)) {
#pragma unroll
          for (int q = 0; q < kGroupBatch; ++q) {
            // group i of this wave is column group cg = wv + 4 i (columns 16 cg ..)
            const int i = bd * kGroupBatch + q;
            const bool in = i < ncg;
            const int cg = wv + 4 * (in ? i : 0);
            const uint32_t off =
                pk ? (uint32_t)(((cg / 16) * nst2 + j) * kPkBlock + ((cg % 16) * 16 + lr) * 64 + 16 * lg)
                   : doff0 + (uint32_t)((int64_t)cg * 16 * I * WSZ);
            D.b[q] = load_w<FP8>(w2r, in ? off : kNoOperand, 0);
            if constexpr (FP8) D.s[q] = g.s2[sd0 + (int64_t)(cg * 16 / 128) * (I / 128)];
          }
        };
        DownBatch<FP8> D0, D1;
        load_down(D0, 0);
        // g (wave matrix 0) and u (1) of rows 4 lg + c of each group, column
        // 16 half + lr of the slice
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
          for (int c = 0; c < 4; ++c) s_gu[mt][gi * 16 + 4 * lg + c][half * 16 + lr] = acc[gi][c];
        __syncthreads();
        {
          // 32 rows x 32 columns: 4 consecutive columns per thread
          const int row = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * 4;
          if (row < 16 * NG) {
            u32x2 o;
#pragma unroll
            for (int q = 0; q < 2; ++q)
              o[q] = bf16_pair(silu_times(s_gu[0][row][c0 + 2 * q], s_gu[1][row][c0 + 2 * q]),
                               silu_times(s_gu[0][row][c0 + 2 * q + 1], s_gu[1][row][c0 + 2 * q + 1]));
            *(u32x2*)&s_h[row][c0] = o;
          }
        }
        __syncthreads();

        // ---- down over the slice: y_j[rows][H] ----
        bf16x8 ha[NG];  // [row group]: the 32-deep slice
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) ha[gi] = *(const bf16x8*)&s_h[gi * 16 + lr][8 * lg];
        int slot_of[NG][4];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
          for (int c = 0; c < 4; ++c) slot_of[gi][c] = s_slot[gi * 16 + 4 * lg + c];
        float* prow = g.part + (int64_t)j * g.slots * H;
        auto mul_down = [&](const DownBatch<FP8>& D, int bd) __attribute__((always_inline)) {
#pragma unroll
          for (int q = 0; q < kGroupBatch; ++q) {
            const int i = bd * kGroupBatch + q;
            const bf16x8 b = decode<FP8>(D.b[q], FP8 ? D.s[q] : 1.0f);
            f32x4 y[NG];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) y[gi] = mfma(ha[gi], b, f32x4{0.f, 0.f, 0.f, 0.f});
            if (i >= ncg) continue;
            const int col = (wv + 4 * i) * 16 + lr;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
              for (int c = 0; c < 4; ++c)
                if (slot_of[gi][c] >= 0) prow[(int64_t)slot_of[gi][c] * H + col] = y[gi][c];
          }
        };
        for (int bd = 0; bd < nbd; bd += 2) {
          load_down(D1, bd + 1);
          mul_down(D0, bd);
          load_down(D0, bd + 2);
          mul_down(D1, bd + 1);
        }
      };
      if (s_slot[16] < 0)
        pass(std::integral_constant<int, 1>{});
      else
        pass(std::integral_constant<int, 2>{});
    }
  }
}

// The combine of the fused plan.  A workgroup takes one token and 32 columns: 8
// column vectors of 4 floats x 32 pair lanes.  The token's (slot i, slice j)
// pairs, numbered p = i * nsl + j, are dealt to the lanes (lane l: p = l, l + 32,
// ... in ascending order); a lane adds topk_w[t][i] * part[j][t k + i] over its
// pairs, loading eight pairs before it adds them, and skips the slots of other
// GPUs' experts.  The 32 lane sums are then added in lane order through LDS and
// rounded to bf16 once: a fixed order, so y is deterministic.  With a nonzero
// device status the FFN may have skipped rows, and y is written as zeros.
constexpr int kCombLanes = 32;
constexpr int kCombVecs = 256 / kCombLanes;  // column vectors of 4 floats per workgroup
constexpr int kCombBatch = 8;  // pairs loaded before they are added

__global__ void __launch_bounds__(256) combine_fused_kernel(const float* __restrict__ part,
                                                            const int32_t* __restrict__ status,
                                                            const int32_t* __restrict__ slot_pos,
                                                            const float* __restrict__ w,
                                                            uint16_t* __restrict__ y, int B, int H,
                                                            int k, int nsl, int slots) {
  __shared__ f32x4 red[kCombLanes][kCombVecs];
  __shared__ float s_w[32];  // the token's router weights; 0 for other GPUs' experts
  const int cv = threadIdx.x % kCombVecs, sl = threadIdx.x / kCombVecs;
  const bool ok = *status == MOE_DEV_OK;
  const int chunks = H / (4 * kCombVecs);
  const int pairs = k * nsl;
  for (int64_t item = blockIdx.x; item < (int64_t)B * chunks; item += gridDim.x) {
    const int t = (int)(item / chunks);
    const int col = (int)(item - (int64_t)t * chunks) * (4 * kCombVecs) + cv * 4;
    __syncthreads();  // the previous item's readers of s_w and red are done
    if (threadIdx.x < k) s_w[threadIdx.x] = slot_pos[t * k + threadIdx.x] >= 0 ? w[t * k + threadIdx.x] : 0.f;
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (ok) {
      for (int p0 = sl; p0 < pairs; p0 += kCombLanes * kCombBatch) {
        f32x4 v[kCombBatch];
        float g[kCombBatch];
#pragma unroll
        for (int q = 0; q < kCombBatch; ++q) {
          const int pq = p0 + q * kCombLanes;
          const int i = pq / nsl, j = pq - (pq / nsl) * nsl;
          g[q] = pq < pairs ? s_w[i] : 0.f;
          v[q] = g[q] != 0.f ? *(const f32x4*)(part + ((int64_t)j * slots + t * k + i) * H + col)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int q = 0; q < kCombBatch; ++q)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] = __builtin_fmaf(g[q], v[q][c], acc[c]);
      }
    }
    red[sl][cv] = acc;
    __syncthreads();
    if (sl == 0) {
      f32x4 tot = red[0][cv];
#pragma unroll
      for (int q = 1; q < kCombLanes; ++q) tot += red[q][cv];
      u32x2 o = {bf16_pair(tot[0], tot[1]), bf16_pair(tot[2], tot[3])};
      *(u32x2*)(y + (int64_t)t * H + col) = o;
    }
  }
}

}  // namespace

int64_t fused_ws_bytes(const moe_problem& p) {
  return 256 + (int64_t)(p.inter / kSlice) * p.tokens * p.top_k * p.hidden * 4;
}

hipError_t launch_fused_ffn(const moe_problem& p, const void* x, const void* w1, const void* w3,
                            const void* w2, const float* s1, const float* s3, const float* s2,
                            const int32_t* sorted_slots, const int32_t* block_expert,
                            const int32_t* num_blocks, const int32_t* variant, void* ws,
                            int num_cus, int64_t rows_max, hipStream_t s) {
  FusedArgs g;
  g.x = x;
  g.w1 = w1;
  g.w3 = w3;
  g.w2 = w2;
  g.s1 = s1;
  g.s3 = s3;
  g.s2 = s2;
  g.sorted_slots = sorted_slots;
  g.block_expert = block_expert;
  g.num_blocks = num_blocks;
  g.variant = variant;
  g.status = (int32_t*)ws;
  g.wpk = p.weight_dtype == MOE_BF16 ? (const uint8_t*)p.packed_weights : nullptr;
  g.part = (float*)((char*)ws + 256);
  g.H = p.hidden;
  g.I = p.inter;
  g.k = p.top_k;
  g.E_loc = p.local_experts;
  g.slots = p.tokens * p.top_k;
  g.rows_max = rows_max;
  // row-blocks: at most ceil(slots / 16) + one partial block per active expert
  const int64_t slots = g.slots;
  const int64_t nb_max = (slots + kMinBlockM - 1) / kMinBlockM + (p.local_experts < slots ? p.local_experts : slots);
  const int64_t tiles = nb_max * (p.inter / kSlice);
  // up to four workgroups per CU at once: every tile of a small batch in flight
  const int64_t cap = 4 * (int64_t)num_cus;
  const int grid = (int)(tiles < cap ? tiles : cap);
  if (p.weight_dtype == MOE_FP8_E4M3)
    fused_ffn_kernel<true><<<grid, kFusedThreads, 0, s>>>(g);
  else
    fused_ffn_kernel<false><<<grid, kFusedThreads, 0, s>>>(g);
  return hipGetLastError();
}

hipError_t launch_combine_fused(const moe_problem& p, const void* ws, const int32_t* slot_pos,
                                const float* w, void* y, hipStream_t s) {
  const int64_t items = (int64_t)p.tokens * (p.hidden / (4 * kCombVecs));
  const int grid = (int)(items < 8192 ? items : 8192);
  combine_fused_kernel<<<grid, 256, 0, s>>>((const float*)((const char*)ws + 256), (const int32_t*)ws,
                                            slot_pos, w, (uint16_t*)y, p.tokens, p.hidden,
                                            p.top_k, p.inter / kSlice, p.tokens * p.top_k);
  return hipGetLastError();
}

}  // namespace moe
