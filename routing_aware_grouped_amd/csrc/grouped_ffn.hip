// grouped_ffn.hip -- step 4: the polymorphic grouped expert FFN.
//
// For each padded row r of the expert grouping (expert e = block_expert[r / b]):
//   phase 1:  h[r] = silu(x[t] W1_e^T) * (x[t] W3_e^T),  t = sorted_slots[r] / k
//   phase 2:  y_slots[r] = h[r] W2_e^T
// (GC-MoE arXiv 2611.04222, 2.1 Eq. 1: W1 stacks gate and up, W2 is the down
// projection; RaMP arXiv 2604.26039, 2.1: each expert is a gated MLP.)  Padding rows
// (sorted_slots = -1) read zeros and so produce zeros.
//
// Polymorphism (RaMP 3.3): every compiled tile configuration lives in one kernel per
// phase.  Each workgroup reads the chosen index and the row-block count from device
// memory and runs that configuration's tiles, so the launch shape is fixed and the
// choice needs neither a host round trip nor a new launch.  The grid is persistent
// (compute units x workgroups per unit, capped by the largest tile count any
// configuration can produce); workgroups stride over the chosen configuration's
// tiles.  All configurations share one 256-thread workgroup shape, one LDS budget
// and one register allocation (one occupancy class).
//
// Tile order: the tile index runs over row-blocks fastest, so consecutive tiles
// reuse one expert's weight panel; workgroup ids are remapped so that consecutive
// tiles land on the same XCD (the hardware deals workgroups round-robin over the 8
// XCDs, each with its own L2).
//
// Math: bf16 (and fp8-decoded) operands on v_mfma_f32_16x16x32_bf16, fp32
// accumulation; the fp32 problem uses v_mfma_f32_16x16x4_f32 over the same k=32
// fragments.  Rows are tokens (the MFMA A operand), columns are weight rows (B
// operand), both K-contiguous in memory, so each lane's 8-element fragment is one
// 16-byte (bf16), 8-byte (fp8) or 32-byte (f32) contiguous load.  FP8 E4M3FN weights
// are decoded with the hardware converter, multiplied by their 128x128 block scale
// in fp32 and rounded to bf16 (w = q * s).
//
// Configurations (BLOCK_M x BLOCK_N per workgroup; waves M x N x K-split):
//   small tiles stream weights straight from HBM into registers with a multi-step
//   software prefetch; waves that split K inside a tile are summed through LDS in a
//   fixed order, so results are deterministic.
#include "moe_common.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// operand fragments: 8 consecutive k of one row, per lane
// ---------------------------------------------------------------------------
template <bool F32>
struct Frag;
template <>
struct Frag<false> {
  bf16x8 v;
};
template <>
struct Frag<true> {
  f32x4 lo, hi;
};

__device__ __forceinline__ void zero_frag(Frag<false>& f) {
  u32x4 z = {0u, 0u, 0u, 0u};
  f.v = __builtin_bit_cast(bf16x8, z);
}
__device__ __forceinline__ void zero_frag(Frag<true>& f) {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f.lo = z;
  f.hi = z;
}

__device__ __forceinline__ void mma(f32x4& acc, const Frag<false>& a, const Frag<false>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<true>& a, const Frag<true>& b) {
  // lane l holds k = 8*(l/16) + c in element c; the c-th 16x16x4 product sums
  // k = {c, 8+c, 16+c, 24+c}, so the eight products cover k = 0..31 once.
#pragma unroll
  for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[c], b.lo[c], acc, 0, 0, 0);
#pragma unroll
  for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[c], b.hi[c], acc, 0, 0, 0);
}

// 16-byte / 32-byte loads of 8 elements starting at p (element index already applied)
__device__ __forceinline__ void load_frag(Frag<false>& f, const uint16_t* p) {
  f.v = __builtin_bit_cast(bf16x8, *(const u32x4*)p);
}
__device__ __forceinline__ void load_frag(Frag<true>& f, const float* p) {
  f.lo = *(const f32x4*)p;
  f.hi = *(const f32x4*)(p + 4);
}

// fp8 E4M3FN x8 (8 bytes) * scale -> bf16 x8
__device__ __forceinline__ void fp8_to_frag(Frag<false>& f, u32x2 q, float s) {
  u32x4 o;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(q[h], false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(q[h], true);
    o[2 * h] = pack_bf16x2(a[0] * s, a[1] * s);
    o[2 * h + 1] = pack_bf16x2(b[0] * s, b[1] * s);
  }
  f.v = __builtin_bit_cast(bf16x8, o);
}

// ---------------------------------------------------------------------------
// element types per problem
// ---------------------------------------------------------------------------
enum WKind { W_F32 = 0, W_BF16 = 1, W_FP8 = 2 };

template <int WK_>
struct Types;
template <>
struct Types<W_F32> {
  using Act = float;
  using Wt = float;
  static constexpr bool F32 = true;
};
template <>
struct Types<W_BF16> {
  using Act = uint16_t;
  using Wt = uint16_t;
  static constexpr bool F32 = false;
};
template <>
struct Types<W_FP8> {
  using Act = uint16_t;
  using Wt = uint8_t;
  static constexpr bool F32 = false;
};

// load 8 weights of row `row` (of a [rows][K] matrix), k offset kk, for expert
// matrix base w; fp8 applies the block scale of (row/128, kk/128)
// (sidx is wave-uniform: all 64 lanes of a fragment fall in one 128x128 block)
template <int WKIND>
__device__ __forceinline__ void load_w(Frag<Types<WKIND>::F32>& f, const typename Types<WKIND>::Wt* w,
                                       int64_t row, int K, int kk, const float* sc, int64_t sidx) {
  if constexpr (WKIND == W_FP8) {
    const u32x2 q = *(const u32x2*)(w + row * K + kk);
    fp8_to_frag(f, q, sc[sidx]);
  } else {
    load_frag(f, w + row * K + kk);
  }
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) {
  *p = v;
}
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float v) {
  *p = f32_to_bf16_bits(v);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// ---------------------------------------------------------------------------
// kernel arguments
// ---------------------------------------------------------------------------
struct FfnArgs {
  const void* x;   // [B][H] act
  const void* w1;  // [E_loc][I][H]
  const void* w3;  // [E_loc][I][H]
  const void* w2;  // [E_loc][H][I]
  const float* s1;
  const float* s3;
  const float* s2;
  const int32_t* sorted_slots;
  const int32_t* block_expert;
  const int32_t* num_blocks;
  const int32_t* variant;
  void* h;        // [rows_max][I] act
  void* y_slots;  // [rows_max][H] act
  int H, I, k;
  int E_loc;
  int slots;      // B * k
  int64_t rows_max;
};

__device__ __forceinline__ int xcd_tile_slot(int wg, int grid) {
  // consecutive slots on one XCD: the hardware places workgroup wg on XCD wg % 8
  const int per = grid >> 3;
  if (per == 0 || (grid & 7)) return wg;
  return (wg & 7) * per + (wg >> 3);
}

// ---------------------------------------------------------------------------
// one tile configuration, one phase
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int WKS, int PF, int PHASE, int WKIND>
struct TileRunner {
  using T = Types<WKIND>;
  using Act = typename T::Act;
  using Wt = typename T::Wt;
  static constexpr bool F32 = T::F32;
  static constexpr int MW = BM / WM;
  static constexpr int NW = BN / WN;
  static constexpr int FM = MW / 16;
  static constexpr int FN = NW / 16;
  static constexpr int NMAT = PHASE == 1 ? 2 : 1;  // gate and up share the A rows
  static constexpr int NB = PF + 1;                // register ring of k-steps
  static_assert(WM * WN * WKS == 4, "4 waves per workgroup");
  static_assert(FM >= 1 && FN >= 1, "tile too small for the wave layout");

  // LDS floats needed for the in-tile K-split reduction
  static constexpr int kLdsFloats = (WKS > 1) ? (WKS - 1) * WM * WN * NMAT * FM * FN * 4 * 64 : 0;

  struct Step {
    Frag<F32> a[FM];
    Frag<F32> b[NMAT][FN];
  };

  __device__ static void run(const FfnArgs& g, float* lds, int nblocks) {
    const int N = PHASE == 1 ? g.I : g.H;
    const int K = PHASE == 1 ? g.H : g.I;
    const int tiles_n = N / BN;
    const int total = nblocks * tiles_n;
    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x & 63;
    const int wk = wave % WKS;
    const int wn = (wave / WKS) % WN;
    const int wm = wave / (WKS * WN);
    const int lr = lane & 15;         // row (A) / column (B) inside a 16-block
    const int lk = (lane >> 4) * 8;   // k offset of this lane inside a 32-chunk
    const int nks = K / 32;           // k-steps of 32
    const int nsteps = nks > wk ? (nks - wk + WKS - 1) / WKS : 0;
    const Wt* wmat0 = (const Wt*)(PHASE == 1 ? g.w1 : g.w2);
    const Wt* wmat1 = (const Wt*)(PHASE == 1 ? g.w3 : g.w2);
    const float* smat0 = PHASE == 1 ? g.s1 : g.s2;
    const float* smat1 = PHASE == 1 ? g.s3 : g.s2;
    const int Kb = K / 128;  // scale blocks along K
    const int Nb = N / 128;

    for (int tile = xcd_tile_slot(blockIdx.x, gridDim.x); tile < total; tile += gridDim.x) {
      const int rb = tile % nblocks;  // row-block (fastest: reuse of one weight panel)
      const int nt = tile / nblocks;
      const int e = g.block_expert[rb];
      if ((unsigned)e >= (unsigned)g.E_loc) continue;  // uniform: whole workgroup skips
      const int64_t row0 = (int64_t)rb * BM;
      const int n0 = nt * BN + wn * NW;

      // A rows of this lane: token rows (phase 1, gathered) or h rows (phase 2)
      const Act* arow[FM];
      bool avalid[FM];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int64_t r = row0 + wm * MW + fm * 16 + lr;
        if (PHASE == 1) {
          const int s = g.sorted_slots[r];
          avalid[fm] = s >= 0 && s < g.slots;  // anything else is a padding row
          arow[fm] = (const Act*)g.x + (int64_t)(s >= 0 ? s / g.k : 0) * K;
        } else {
          avalid[fm] = true;
          arow[fm] = (const Act*)g.h + r * K;
        }
      }
      // B rows of this lane: weight rows n of expert e
      int64_t brow[FN];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) brow[fn] = (int64_t)e * N + n0 + fn * 16 + lr;
      // fp8 scale index base per fragment (all 64 lanes share one 128x128 block)
      int64_t sbase[FN];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) sbase[fn] = ((int64_t)e * Nb + (n0 + fn * 16) / 128) * Kb;

      f32x4 acc[NMAT][FM][FN];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

      Step buf[NB];
      auto load_step = [&](Step& st, int step) {
        const int kk0 = (wk + step * WKS) * 32;  // wave-uniform
        const int kk = kk0 + lk;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          if (avalid[fm])
            load_frag(st.a[fm], arow[fm] + kk);
          else
            zero_frag(st.a[fm]);
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          load_w<WKIND>(st.b[0][fn], wmat0, brow[fn], K, kk, smat0, sbase[fn] + kk0 / 128);
          if (NMAT == 2)
            load_w<WKIND>(st.b[NMAT - 1][fn], wmat1, brow[fn], K, kk, smat1, sbase[fn] + kk0 / 128);
        }
      };
      auto compute_step = [&](const Step& st) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) mma(acc[m][i][j], st.a[i], st.b[m][j]);
      };

#pragma unroll
      for (int u = 0; u < PF; ++u)
        if (u < nsteps) load_step(buf[u], u);
      for (int base = 0; base < nsteps; base += NB) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int step = base + u;
          if (step < nsteps) {
            if (step + PF < nsteps) load_step(buf[(u + PF) % NB], step + PF);
            compute_step(buf[u]);
          }
        }
      }

      // in-tile K-split: waves wk > 0 hand their partial sums to wave wk = 0
      if constexpr (WKS > 1) {
        const int slot_base = ((wm * WN + wn) * (WKS - 1)) * NMAT * FM * FN * 4 * 64;
        if (wk > 0) {
          float* dst = lds + slot_base + (wk - 1) * NMAT * FM * FN * 4 * 64;
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                  dst[(((m * FM + i) * FN + j) * 4 + c) * 64 + lane] = acc[m][i][j][c];
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll
          for (int q = 0; q < WKS - 1; ++q) {
            const float* src = lds + slot_base + q * NMAT * FM * FN * 4 * 64;
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
              for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                  for (int c = 0; c < 4; ++c)
                    acc[m][i][j][c] += src[(((m * FM + i) * FN + j) * 4 + c) * 64 + lane];
          }
        }
        __syncthreads();
        if (wk != 0) continue;
      }

      // epilogue: lane holds rows 4*(lane/16)+c, column lane%16 of each 16x16 block
      Act* out = (Act*)(PHASE == 1 ? g.h : g.y_slots);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int64_t r = row0 + wm * MW + i * 16 + (lane >> 4) * 4 + c;
            const int n = n0 + j * 16 + lr;
            float v;
            if (PHASE == 1)
              v = silu_mul(acc[0][i][j][c], acc[NMAT - 1][i][j][c]);
            else
              v = acc[0][i][j][c];
            store_out<Act>(out + r * N + n, v);
          }
    }
  }
};

// configuration table: must match kVariants in moe_common.h
template <int V, int PHASE, int WKIND>
struct Cfg;
#define MOE_CFG(V, BM, BN1, BN2, WM, WN, WKS, PF)                                           \
  template <int PHASE, int WKIND>                                                         \
  struct Cfg<V, PHASE, WKIND> {                                                           \
    using R = TileRunner<BM, (PHASE == 1 ? BN1 : BN2), WM, WN, WKS, PF, PHASE, WKIND>;    \
  };                                                                                      \
  static_assert(kVariants[V].bm == BM && kVariants[V].bn1 == BN1 && kVariants[V].bn2 == BN2 && \
                    kVariants[V].wm == WM && kVariants[V].wn == WN && kVariants[V].wk == WKS &&  \
                    kVariants[V].splitk == 1 && kVariants[V].bk == 32 * WKS,                    \
                "kernel configuration table out of sync with kVariants");
MOE_CFG(0, 16, 16, 16, 1, 1, 4, 3)
MOE_CFG(1, 32, 32, 32, 1, 2, 2, 2)
MOE_CFG(2, 64, 64, 64, 2, 2, 1, 1)
MOE_CFG(3, 128, 64, 128, 2, 2, 1, 1)
#undef MOE_CFG

template <int PHASE, int WKIND>
constexpr int lds_floats() {
  int m = 1;
  m = Cfg<0, PHASE, WKIND>::R::kLdsFloats > m ? Cfg<0, PHASE, WKIND>::R::kLdsFloats : m;
  m = Cfg<1, PHASE, WKIND>::R::kLdsFloats > m ? Cfg<1, PHASE, WKIND>::R::kLdsFloats : m;
  m = Cfg<2, PHASE, WKIND>::R::kLdsFloats > m ? Cfg<2, PHASE, WKIND>::R::kLdsFloats : m;
  m = Cfg<3, PHASE, WKIND>::R::kLdsFloats > m ? Cfg<3, PHASE, WKIND>::R::kLdsFloats : m;
  return m;
}

template <int PHASE, int WKIND>
__global__ void __launch_bounds__(kThreads) ffn_phase_kernel(FfnArgs g) {
  __shared__ float lds[lds_floats<PHASE, WKIND>()];
  const int v = *g.variant;
  int nb = *g.num_blocks;
  if (nb <= 0 || v < 0 || v >= kNumVariants) return;
  // never address rows beyond the buffers, whatever the device state says
  const int nb_cap = (int)(g.rows_max / kVariants[v].bm);
  nb = nb < nb_cap ? nb : nb_cap;
  switch (v) {
    case 0: Cfg<0, PHASE, WKIND>::R::run(g, lds, nb); break;
    case 1: Cfg<1, PHASE, WKIND>::R::run(g, lds, nb); break;
    case 2: Cfg<2, PHASE, WKIND>::R::run(g, lds, nb); break;
    case 3: Cfg<3, PHASE, WKIND>::R::run(g, lds, nb); break;
    default: break;  // out-of-range index: align_sort already produced no rows
  }
}

template <int WKIND>
hipError_t launch_w(const FfnArgs& g, int grid1, int grid2, hipStream_t s) {
  ffn_phase_kernel<1, WKIND><<<grid1, kThreads, 0, s>>>(g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ffn_phase_kernel<2, WKIND><<<grid2, kThreads, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_ffn(const moe_problem& p, const void* x, const void* w1,
                              const void* w3, const void* w2, const float* s1, const float* s3,
                              const float* s2, const int32_t* sorted_slots,
                              const int32_t* block_expert, const int32_t* num_blocks,
                              const int32_t* variant, void* y_slots, void* h, int num_cus,
                              int64_t rows_max, hipStream_t s) {
  FfnArgs g{x, w1, w3, w2, s1, s3, s2, sorted_slots, block_expert, num_blocks, variant,
            h, y_slots, p.hidden, p.inter, p.top_k, p.local_experts, p.tokens * p.top_k,
            rows_max};
  // persistent grid: compute units x workgroups per unit, capped by the most tiles
  // any configuration can produce for this problem
  int64_t max_t1 = 0, max_t2 = 0;
  for (int v = 0; v < kNumVariants; ++v) {
    const int64_t rb = rows_max / kVariants[v].bm;
    const int64_t t1 = rb * (p.inter / kVariants[v].bn1);
    const int64_t t2 = rb * (p.hidden / kVariants[v].bn2);
    max_t1 = t1 > max_t1 ? t1 : max_t1;
    max_t2 = t2 > max_t2 ? t2 : max_t2;
  }
  int64_t g1 = (int64_t)num_cus * kWgPerCuPhase1, g2 = (int64_t)num_cus * kWgPerCuPhase2;
  g1 = g1 < max_t1 ? g1 : max_t1;
  g2 = g2 < max_t2 ? g2 : max_t2;
  if (g1 < 1) g1 = 1;
  if (g2 < 1) g2 = 1;
  switch (p.weight_dtype) {
    case MOE_F32: return launch_w<W_F32>(g, (int)g1, (int)g2, s);
    case MOE_BF16: return launch_w<W_BF16>(g, (int)g1, (int)g2, s);
    case MOE_FP8_E4M3: return launch_w<W_FP8>(g, (int)g1, (int)g2, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
