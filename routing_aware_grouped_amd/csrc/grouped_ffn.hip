// grouped_ffn.hip -- the polymorphic, persistent grouped expert FFN (one kernel,
// launched once for the gate/up GEMM and once for the down GEMM).
//
// What is computed, for every padded row r of the expert grouping with
// e = block_expert[r / b] and t = sorted_slots[r] / k (GC-MoE arXiv 2611.04222,
// section 2.1, Eq. 1: W1 stacks gate and up, W2 is the down projection; RaMP arXiv
// 2604.26039, section 2.1: each expert is a gated MLP):
//   gate/up phase:  h[r]       = silu(x[t] W1_e^T) * (x[t] W3_e^T)
//   down phase:     y_slots[r] = h[r] W2_e^T
// Padding rows (sorted_slots = -1) are neither read nor written.
//
// Polymorphism (RaMP section 3.3 and appendix A.8): every compiled tile
// configuration lives in this one kernel.  Each workgroup reads the chosen index
// and the row-block count from device memory and runs that configuration, so the
// launch shape is fixed and the choice needs no host round trip.  All
// configurations share one workgroup size, one LDS allocation and one register
// budget (one occupancy class).
//
// Scheduling.  The two GEMM phases are two launches of this kernel (the down
// phase needs every column of h for its row-block, and a dependency between
// workgroups of one launch would need a wait); each launch is persistent
// (compute units x kWgPerCu workgroups) and deals its tiles out statically:
// tiles are numbered in chunks of 16 column tiles, row-block slowest inside a
// chunk (Tile::tile_rc), tile t goes to slot t mod G, and slots are numbered so
// that G / 8 consecutive ones sit on one XCD (the hardware deals workgroup ids
// round-robin over the 8 XCDs, each with its own L2): the tiles that run together
// on one XCD share a few row-blocks of token rows and many weight slices.  There are no atomics and
// no waits between workgroups; every loop has a static bound.
//
// Data movement.  Each pipeline stage covers BK elements of the reduction for the
// tile's A rows (tokens, or h rows) and its weight rows.  Threads load 16-byte
// chunks so that consecutive lanes read consecutive bytes of one row (a wave
// instruction reads 1 KiB of contiguous rows: full cache lines, the pattern that
// streams HBM fastest), hold them in registers RS stages ahead, and write them to
// a double-buffered LDS tile.  LDS rows are XOR-swizzled in 16-byte units so that
// the MFMA fragment reads (16 rows x 16 bytes per quarter wave) are conflict free.
// FP8 E4M3FN weights are decoded once, while staging: w = q * s with the 128 x 128
// block scale in fp32, rounded to bf16 (RaMP section 3.3's block-scaled FP8).
//
// Math.  v_mfma_f32_16x16x32_bf16 for bf16 operands (fp8 weights decoded to
// bf16), v_mfma_f32_16x16x4_f32 for the fp32 problem; fp32 accumulation.  On the
// FP8 activation path the gate/up phase stages fp8 x and fp8 weights unchanged and
// multiplies them with v_mfma_f32_16x16x128_f8f6f4: each instruction covers one
// 128-deep block, whose activation scale (per row) and weight scale (per tile)
// multiply its sums before they are added (the block-scaled FP8 GEMM of RaMP
// section 3.3 and appendix A.8).  Waves
// are arranged WM x WN x WK over the tile; waves that split K inside a tile add
// their partial sums through LDS in a fixed order, so results are deterministic.
#include <type_traits>

#include "moe_common.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// element types
// ---------------------------------------------------------------------------
enum WKind { W_F32 = 0, W_BF16 = 1, W_FP8 = 2, W_FP8A = 3 };

template <int WK_>
struct Types;
// Act: the A operand (x or h) as read; Out: the phase's output (h or y_slots)
template <>
struct Types<W_F32> {
  using Act = float;
  using Wt = float;
  using Out = float;
  static constexpr int asz = 4, wsz = 4;
};
template <>
struct Types<W_BF16> {
  using Act = uint16_t;
  using Wt = uint16_t;
  using Out = uint16_t;
  static constexpr int asz = 2, wsz = 2;
};
template <>
struct Types<W_FP8> {
  using Act = uint16_t;
  using Wt = uint8_t;
  using Out = uint16_t;
  static constexpr int asz = 2, wsz = 1;
};
// FP8 activation path: fp8 x or h (one fp32 scale per row and 128 columns), fp8
// weights, bf16 output (h or y_slots)
template <>
struct Types<W_FP8A> {
  using Act = uint8_t;
  using Wt = uint8_t;
  using Out = uint16_t;
  static constexpr int asz = 1, wsz = 1;
};

// MFMA operand fragment: 8 consecutive k of one row per lane
template <int KIND>
struct Frag {  // bf16 operands (also fp8 weights decoded to bf16)
  bf16x8 v;
};
template <>
struct Frag<W_F32> {
  f32x4 lo, hi;
};
template <>
struct Frag<W_FP8A> {  // 32 fp8 values of one row: a 128-deep block over 4 lanes
  u32x4 lo, hi;
};
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

template <int KIND>
__device__ __forceinline__ void mma(f32x4& acc, const Frag<KIND>& a, const Frag<KIND>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
// fp8 x fp8 over one 128-deep block, from zero: both operands E4M3 (format 0) and
// unit block exponents (127 = 2^0), so the instruction is a plain fp8 product
__device__ __forceinline__ f32x4 mma_fp8_block(const Frag<W_FP8A>& a, const Frag<W_FP8A>& b) {
  const i32x8 av = __builtin_bit_cast(i32x8, __builtin_shufflevector(a.lo, a.hi, 0, 1, 2, 3, 4, 5, 6, 7));
  const i32x8 bv = __builtin_bit_cast(i32x8, __builtin_shufflevector(b.lo, b.hi, 0, 1, 2, 3, 4, 5, 6, 7));
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                          0, 127, 0, 127);
}
template <>
__device__ __forceinline__ void mma<W_F32>(f32x4& acc, const Frag<W_F32>& a, const Frag<W_F32>& b) {
  // lane l holds k = 8*(l/16) + c in element c; the c-th 16x16x4 product sums
  // k = {c, 8+c, 16+c, 24+c}, so the eight products cover k = 0..31 once.
#pragma unroll
  for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[c], b.lo[c], acc, 0, 0, 0);
#pragma unroll
  for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[c], b.hi[c], acc, 0, 0, 0);
}

// Buffer resource of `bytes` bytes from `base` for untyped buffer loads (the last
// descriptor word selects 32-bit data, as gfx9-family untyped loads need).  A load
// whose offset is at or past `bytes` returns zeros and touches no memory; kOob is
// past every range the host allows (each operand buffer is below 2^31 bytes).
constexpr uint32_t kOob = 0x80000000u;
constexpr int kCacheNt = 2;  // cache-policy operand of a buffer load: non-temporal
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// LDS row swizzle in 16-byte units for rows of C chunks: chunk c of row r sits at
// c ^ ((r >> 1) & 3) for 64-byte rows, c ^ (r & 7) for 128-byte rows and
// c ^ (r & 15) for longer ones.  A stage write covers each row's chunks once.
// The choice is measured, not derived: with rocprofv3 on gfx950, fragment reads
// (ds_read_b128, 16 consecutive rows per quarter wave, one logical chunk) show no
// bank-conflict cycles with these swizzles.  For 64-byte rows the swizzles on
// row bits 2-3 or 0-1, or none, double the LDS cycles of a read (half of them
// conflicts); for 256-byte rows c ^ ((r >> 1) & 15) does the same and no swizzle
// makes 87% of the cycles conflicts.
template <int C>
__device__ __forceinline__ int swz(int row) {
  return C == 4 ? (row >> 1) & 3 : row & (C >= 16 ? 15 : 7);
}

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

// 16 fp8 E4M3FN codes times one scale -> 16 bf16 (two 16-byte LDS chunks)
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4& q, float s, u32x4& o0, u32x4& o1) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(q[w], false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(q[w], true);
    const uint32_t p0 = pack2_bf16(a[0] * s, a[1] * s);
    const uint32_t p1 = pack2_bf16(b[0] * s, b[1] * s);
    if (w < 2) {
      o0[2 * w] = p0;
      o0[2 * w + 1] = p1;
    } else {
      o1[2 * (w - 2)] = p0;
      o1[2 * (w - 2) + 1] = p1;
    }
  }
}

// silu(g) * u = g / (1 + e^-g) * u, with the hardware reciprocal (about 1 ulp):
// the IEEE divide took about ten instructions per output, a large share of the
// tile epilogue, for accuracy far below the bf16 output's rounding.  Large
// negative g: e^-g -> inf, its reciprocal 0, the product 0 (the limit).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) {
  *p = v;
}
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float v) {
  *p = __builtin_bit_cast(uint16_t, (__bf16)v);
}

// ---------------------------------------------------------------------------
// kernel arguments and the tile queue
// ---------------------------------------------------------------------------
struct FfnArgs {
  const void* x;   // [B][H] act (the fp8 codes on the FP8 activation path)
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
  void* h;         // [rows_max][I] act
  void* y_slots;   // [rows_max][H] act
  float* part;     // [grid][2][NMAT * BM * BN] fp32 sums of split tail tiles
  int H, I, k;
  int E_loc;
  int slots;  // B * k
  int64_t rows_max;
  const float* xs;  // [B][H/128] activation scales of the FP8 activation path
  int n_shared;     // shared experts (row-blocks after the routed ones)
  int32_t* status;  // device status word (MOE_DEV_* bits)
  int grid_stream;  // workgroups of the streaming class's launch (its fix-up needs it)
  const uint8_t* wpk;  // the wide configuration's packed bf16 weights (moe_pack_wide), or null
};

// ring slots of per-tile metadata (see Tile::run_all)
constexpr int kMetaSlots = 4;
// entries of the wide class's first-row-block-per-expert table (local plus shared
// experts, and one past the last); more experts fall back to tile_rc's order
constexpr int kRunTable = 1088;

// slot of workgroup wg so that consecutive slots share an XCD (workgroup wg runs
// on XCD wg % 8)
__device__ __forceinline__ int xcd_slot(int wg, int grid) {
  if (grid & 7) return wg;
  return (wg & 7) * (grid >> 3) + (wg >> 3);
}

// ---------------------------------------------------------------------------
// one tile configuration of one phase
//   BM x BN tile (BN weight rows per matrix; the gate/up phase has two matrices),
//   ROWB = LDS bytes per tile row per stage, waves WM x WN x WK, RS register
//   stages in flight, NT = 64 WM WN WK threads per workgroup; WIDE: the wide
//   class (one workgroup per CU), else the streaming class (two per CU).
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int WK, int ROWB, int RS, int STREAM, int PHASE, int WKIND,
          int NT, bool WIDE>
struct Tile {
  using T = Types<WKIND>;
  using Act = typename T::Act;
  using Wt = typename T::Wt;
  using Out = typename T::Out;
  static constexpr bool F32 = WKIND == W_F32;
  static constexpr bool FP8 = WKIND == W_FP8;    // fp8 weights decoded to bf16
  static constexpr bool FP8A = WKIND == W_FP8A;  // fp8 x fp8
  using FragT = Frag<F32 ? W_F32 : (FP8A ? W_FP8A : W_BF16)>;
  static constexpr int ASZ = T::asz, WSZ = T::wsz;
  static constexpr int NMAT = PHASE == 1 ? 2 : 1;
  static constexpr int BK = ROWB / ASZ;  // reduction elements per stage
  static constexpr int C = ROWB / 16;    // 16-byte LDS chunks per row
  static constexpr int ROWS = BM + NMAT * BN;
  // FP8 activation path: 128-deep scale blocks per stage, and the stage's scales
  // in LDS after its rows: x scales [KB][BM], weight scales [NMAT][KB], 1 spare
  static constexpr int KB = FP8A ? ROWB / 128 : 0;
  // weight-scale blocks (128 output rows each) per matrix that a tile spans
  static constexpr int NSB = BN > 128 ? BN / 128 : 1;
  static constexpr int SC_FLOATS = FP8A ? BM * KB + NMAT * NSB * KB + 1 : 0;
  static constexpr int SC_BYTES = (SC_FLOATS * 4 + 15) / 16 * 16;
  static constexpr int STAGE = ROWS * ROWB + SC_BYTES;  // LDS bytes per stage
  static constexpr int EPC_A = 16 / ASZ;     // elements per global A chunk
  static constexpr int EPC_B = 16 / WSZ;     // elements per global weight chunk
  static constexpr int GCA = BK / EPC_A;     // global chunks per A row per stage
  static constexpr int GCB = BK / EPC_B;     // global chunks per weight row per stage
  static constexpr int GA = BM * GCA;
  static constexpr int GB = NMAT * BN * GCB;
  static constexpr int NA = (GA + NT - 1) / NT;
  static constexpr int NB = (GB + NT - 1) / NT;
  static constexpr int MW = BM / WM, NW = BN / WN;
  static constexpr int FM = MW / 16, FN = NW / 16;
  static constexpr int KSTEPS = BK / (FP8A ? 128 : 32);  // MFMA steps per stage
  static constexpr int RED_FLOATS = (WK > 1) ? (WK - 1) * WM * WN * NMAT * FM * FN * 4 * 64 : 0;
  static constexpr int NFRAG = NMAT * FM * FN;   // 16x16 accumulator blocks per wave
  static constexpr int PIECE = NMAT * BM * BN;   // floats of one partial tile
  static constexpr int LDS_BYTES = 2 * STAGE;
  static constexpr int THREADS = NT;
  static_assert(RED_FLOATS * 4 <= STAGE, "the K-split sums reuse one stage buffer");
  static_assert(WM * WN * WK * 64 == NT, "waves must cover the workgroup");
  static_assert(FM >= 1 && FN >= 1 && MW % 16 == 0 && NW % 16 == 0, "wave tile too small");
  static_assert(C >= 4 && (C & (C - 1)) == 0, "LDS rows must be a power of two of >= 64 bytes");
  static_assert(C >= 8 || !(F32 || FP8A), "fp32 and fp8 x fp8 fragments take 128-byte rows");
  static_assert(KSTEPS % WK == 0, "K-split waves must divide the stage");
  static_assert(!FP8 || GCB * 2 == C, "fp8 chunk pairs");
  static_assert(GA % NT == 0 && GB % NT == 0, "every thread owns whole chunks");
  static_assert((BN * GCB) % NT == 0, "each weight load instruction reads one matrix");
  static_assert(!FP8A || (BM * KB <= NT && NMAT * NSB * KB <= NT && (BN <= 128 ? 128 % BN == 0
                                                                             : BN % 128 == 0) &&
                          (BN / WN) <= 128 && 128 % (BN / WN) == 0),
                "one scale load per thread; a wave's columns share one 128-row weight block");
  // run_all splits the streaming class's tail tiles only (the wide class's bf16
  // down phase splits its own way, in run_dma)
  static constexpr bool SPLITS = !WIDE;
  static_assert(WM * WN * NFRAG * 256 == PIECE && (!SPLITS || PIECE <= kPieceMax),
                "partial tile layout");

  struct Regs {
    u32x4 a[NA];
    u32x4 b[NB];
    float s[FP8 ? NB : 1];
    float xs, ws;  // FP8 activation path: one x scale and one weight scale
  };

  // The LDS swizzle of this tile's rows: swz<C>, except for the fp8 x fp8 tiles'
  // 128-byte rows.  Their fragment read takes two consecutive 16-byte chunks per
  // lane, and with c ^ (r & 7) it measured a quarter of its LDS cycles in bank
  // conflicts on gfx950; c ^ (((r & 3) << 1) | ((r >> 3) & 1)) measured none (the
  // 256- and 512-byte rows' swizzle measured none for this read either).
  __device__ __forceinline__ static int tswz(int row) {
    return (FP8A && C == 8) ? (((row & 3) << 1) | ((row >> 3) & 1)) : swz<C>(row);
  }

  // Tile metadata kept in LDS, in a ring of kMetaSlots slots: the BM slot ids of
  // the tile's rows, the number of leading rows that hold a slot, the local
  // expert, and (wide class) the tile's row-block and column tile.  A slot is
  // refilled at least one barrier after its last reader.
  static constexpr int META = BM + 4;

  // Stores one tile's sums (lane holds rows 4*(lane/16)+c, column lane%16 of each
  // 16x16 block): h = silu(gate) * up in the gate/up phase, y_slots in the down
  // phase.  Rows without a slot (m[r] < 0) are not stored.
  // Component c of an accumulator block that inline-asm MFMAs wrote (run_dma),
  // read by an inline-asm v_accvgpr_read (see store_rows).
  __device__ __forceinline__ static float acc_read(const f32x4& v, int c) {
    float x;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(v[c]));
    return x;
  }
  // store_rows: the same for the NI 16-row groups i0 .. i0 + NI - 1 of the wave.
  // AGPR: the sums are in accumulation registers written by inline-asm MFMAs
  // (run_dma); each is then read by an inline-asm v_accvgpr_read, whose "a"
  // operand keeps every use of the sums in those registers (the compiler makes
  // no copies of them elsewhere, e.g. all 256 at the loop exit), and volatile
  // asm keeps each read after the MFMAs' padding.
  template <int NI, bool AGPR = false>
  __device__ __forceinline__ static void store_rows(const FfnArgs& g, const f32x4 (&acc)[NMAT][NI][FN],
                                                   const int* m, int64_t row0, int n0, int wm,
                                                   int wn, int lane, int i0) {
    auto rd = [&](const f32x4& v, int c) __attribute__((always_inline)) {
      if constexpr (AGPR)
        return acc_read(v, c);
      else
        return v[c];
    };
    const int N = PHASE == 1 ? g.I : g.H;
    const int lr = lane & 15;
    // this lane's first row: one 64-bit base, then wave-uniform row offsets
    const int rl = wm * MW + (lane >> 4) * 4;
    Out* obase = (Out*)(PHASE == 1 ? g.h : g.y_slots) + (row0 + rl) * N + n0 + wn * NW + lr;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int ro = (i0 + i) * 16 + c;
        if (m[rl + ro] < 0) continue;
        Out* orow = obase + ro * N;
#pragma unroll
        for (int jn = 0; jn < FN; ++jn) {
          // a tile of the wide class may reach past N (ragged last column tile)
          if (BN > 128 && n0 + wn * NW + jn * 16 + lr >= N) continue;
          const float v = PHASE == 1 ? silu_mul(rd(acc[0][i][jn], c), rd(acc[NMAT - 1][i][jn], c))
                                     : rd(acc[0][i][jn], c);
          store_out<Out>(orow + jn * 16, v);
        }
      }
  }
  // The direct-load path's tile stores (bf16 out), staged through this wave's
  // LDS tile ost of OSTAGE bytes: each 16-row group of the wave's block is
  // written there row-major (rows padded by 16 bytes), then read back 16 bytes
  // per lane and stored as contiguous row segments.  Direct from the MFMA layout
  // a store instruction wrote 2 bytes per lane to four rows.  The sums are read
  // with acc_read (see store_rows); rows without a slot are not stored, nor
  // columns past N.  The wave's own LDS operations run in order, so the staging
  // tile is rewritten only after the previous group's reads.
  // h of the wide configuration's bf16 tiles (written by the gate/up phase,
  // read by the down phase; workspace only): per row-block rb, per 32-deep block
  // kb of I, 256 rows of 64 bytes, so each down stage reads 16 KiB of
  // consecutive bytes, as from the packed weights.  Byte offset of row-block rb's
  // row 0 at column col (a multiple of 8); row r adds 64 r.
  __device__ __forceinline__ static int64_t hblock_offset(const FfnArgs& g, int64_t rb, int col) {
    return (rb * (g.I / 32) + col / 32) * (256 * 64) + (col % 32) * 2;
  }
  static constexpr int OSTR = NW * 2 + 16;  // staging row stride, bytes
  static constexpr int OSTAGE = 16 * OSTR;  // staging bytes per wave
  __device__ __forceinline__ static void store_staged(const FfnArgs& g, const f32x4 (&acc)[NMAT][FM][FN],
                                                     const int* m, int64_t row0, int n0, int wm,
                                                     int wn, int lane, uint8_t* ost) {
    static_assert(WKIND == W_BF16 && sizeof(Out) == 2 && (NW * 2) % 16 == 0 && 64 % (NW * 2 / 16) == 0,
                  "bf16 rows of whole 16-byte chunks");
    const int N = PHASE == 1 ? g.I : g.H;
    const int lr = lane & 15, lq = lane >> 4;
    constexpr int CPR = NW * 2 / 16;  // 16-byte chunks per staged row
    constexpr int RPI = 64 / CPR;     // rows per read instruction
    const int rr0 = lane / CPR, ch = lane % CPR;
    // gate/up: h in 32-deep blocks per row-block (hblock_offset); down: y_slots rows
    const int col = n0 + wn * NW + ch * 8;
    Out* obase = (Out*)g.y_slots + row0 * N + col;
    uint8_t* hbase = (uint8_t*)g.h + hblock_offset(g, row0 / BM, col);
    const bool col_ok = BN <= 128 || col < N;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int jn = 0; jn < FN; ++jn) {
          const float v = PHASE == 1 ? silu_mul(acc_read(acc[0][i][jn], c), acc_read(acc[NMAT - 1][i][jn], c))
                                     : acc_read(acc[0][i][jn], c);
          *(uint16_t*)(ost + (lq * 4 + c) * OSTR + (jn * 16 + lr) * 2) =
              __builtin_bit_cast(uint16_t, (__bf16)v);
        }
#pragma unroll
      for (int k = 0; k < 16 / RPI; ++k) {
        const int r = k * RPI + rr0;
        const u32x4 d = *(const u32x4*)(ost + r * OSTR + ch * 16);
        const int rr = wm * MW + i * 16 + r;
        if (m[rr] >= 0 && col_ok) {
          if constexpr (PHASE == 1)
            *(u32x4*)(hbase + rr * 64) = d;
          else
            *(u32x4*)(obase + rr * N) = d;
        }
      }
    }
  }
  __device__ __forceinline__ static void store_acc(const FfnArgs& g, const f32x4 (&acc)[NMAT][FM][FN],
                                                  const int* m, int64_t row0, int n0, int wm,
                                                  int wn, int lane) {
    store_rows<FM>(g, acc, m, row0, n0, wm, wn, lane, 0);
  }

  // Tile t of a phase -> row-block rb and column tile nt.  Column tiles come in
  // chunks of kChunk; a chunk holds every row-block's tiles of its columns, the
  // row-block changing slowest.  The G / 8 consecutive tiles that run together on
  // one XCD then cover a few row-blocks (usually of one expert) times many column
  // tiles, so that XCD's L2 serves each token row and each weight slice to many
  // workgroups.
  static constexpr int kChunk = 16;
  __device__ __forceinline__ static void tile_rc(int t, int nb, int ncol, int& rb, int& nt) {
    const int full = ncol / kChunk;
    const int cs = nb * kChunk;
    const int c = t / cs;
    if (c < full) {
      const int l = t - c * cs;
      rb = l / kChunk;
      nt = c * kChunk + l % kChunk;
    } else {  // the last, narrower chunk (t past the last tile: any finite result)
      const int w = ncol > full * kChunk ? ncol - full * kChunk : kChunk;
      const int l = t - full * cs;
      rb = l / w;
      nt = full * kChunk + l % w;
    }
  }

  // Whether the r tail tiles of a phase are split across all G workgroups.  A
  // last round in which at least three quarters of the workgroups stream weights
  // runs near the HBM rate, so streaming configurations split only smaller tails
  // (a split costs the fix-up launch its work, which a small layer cannot hide).
  // The cached configuration splits when the idle share of an unsplit phase,
  // (G - r) / (G (F + 1)) of its time, would exceed one tenth: after several full
  // rounds a nearly full last round costs less than summing its split tiles.
  // The wide class never splits (its tiles are dealt as whole rounds).
  __device__ __forceinline__ static bool split_tail(int r, int G, int F) {
    return SPLITS && r > 0 && (STREAM ? 4 * r < 3 * G : 10 * (G - r) > G * (F + 1));
  }

  // Runs the work of workgroup slot `slot` of `G` (hybrid Stream-K).  The phase's
  // tiles (numbered by tile_rc) come in F = total / G full rounds, dealt
  // round-robin (tiles slot, slot + G, ...).  The r = total - F * G tiles left over would leave
  // most workgroups idle in a last round; when split_tail says so, their r * nst
  // reduction stages are cut into G equal contiguous ranges, one per workgroup, so
  // every workgroup streams the same number of stages to within one (otherwise
  // they are dealt as one more round of whole tiles).  A range spans at most two
  // tail tiles; a tail tile that a range holds only in part is a piece, whose fp32
  // sums go to g.part (two piece slots per workgroup), and the fix-up launch that
  // follows adds the pieces of each split tile in reduction order and stores it.
  // (No workgroup ever waits for another, and no atomics are used.)
  // All the work items (whole tiles, then pieces) form one continuous pipeline, so
  // the next item's first loads are in flight while the current one finishes.
  //
  // SH (shared experts): nb counts the routed row-blocks nbr and then, for each
  // shared expert i, ceil(B / BM) row-blocks of tokens 0..B-1 in order, with
  // local expert index E_loc + i.  Their slot ids are encoded as g.slots + token.
  template <bool SH>
  __device__ __forceinline__ static void run_all(const FfnArgs& g, uint8_t* lds0, uint8_t* lds1,
                                                int* meta3, int nb, int nbr, int slot, int G) {
    const int N = PHASE == 1 ? g.I : g.H;
    const int K = PHASE == 1 ? g.H : g.I;
    const int Btok = g.slots / g.k;
    const int nbs = SH ? (Btok + BM - 1) / BM : 1;  // row-blocks per shared expert
    const int slot_end = SH ? g.slots + Btok : g.slots;
    const int e_end = SH ? g.E_loc + g.n_shared : g.E_loc;
    const int total = nb * ((N + BN - 1) / BN);
    const int nst = (K + BK - 1) / BK;
    const int F = total / G;                        // full rounds
    const int r = total - F * G;                    // tail tiles
    const bool split = split_tail(r, G, F);
    const int Fw = F + (!split && slot < r ? 1 : 0);  // whole tiles of this workgroup
    const int64_t Ut = split ? (int64_t)r * nst : 0;  // tail stages cut into ranges
    const int64_t u0 = (int64_t)slot * Ut / G;      // this workgroup's tail range
    const int len = (int)((int64_t)(slot + 1) * Ut / G - u0);
    const int tp0 = (int)(u0 / nst);                // its first tail tile
    const int sb0 = (int)(u0 - (int64_t)tp0 * nst);  // and the stage it starts at
    const int npc = len == 0 ? 0 : (sb0 + len > nst ? 2 : 1);
    const int nitem = Fw + npc;
    const int nv = Fw * nst + len;  // stages of all items of this workgroup
    if (nv == 0) return;
    // item j: tile, and its stage range [item_sb, item_se)
    auto item_tile = [&](int j) __attribute__((always_inline)) {
      return j < Fw ? slot + j * G : F * G + tp0 + (j - Fw);
    };
    auto item_sb = [&](int j) __attribute__((always_inline)) { return j == Fw ? sb0 : 0; };
    auto item_se = [&](int j) __attribute__((always_inline)) {
      return j < Fw ? nst : (j == Fw ? (sb0 + len < nst ? sb0 + len : nst) : sb0 + len - nst);
    };
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wk = wave % WK;
    const int wn = (wave / WK) % WN;
    const int wm = wave / (WK * WN);
    const Act* abase = (const Act*)(PHASE == 1 ? g.x : g.h);
    const Wt* wmat0 = (const Wt*)(PHASE == 1 ? g.w1 : g.w2);
    const Wt* wmat1 = (const Wt*)(PHASE == 1 ? g.w3 : g.w2);
    const float* smat0 = PHASE == 1 ? g.s1 : g.s2;
    const float* smat1 = PHASE == 1 ? g.s3 : g.s2;

    // ---- tile metadata ----
    // Thread r < BM fetches the slot ids of rows r and r + 1 of a tile (rows that
    // hold a slot come first in a row-block) into registers one pipeline step
    // before they are stored to the tile's ring slot, so the wait for them never
    // drains the stage loads issued in between.
    int ms0 = -1, ms1 = -1, me = -1;
    auto fetch_meta = [&](int j) __attribute__((always_inline)) {
      int rb, nt;
      tile_rc(item_tile(j), nb, (N + BN - 1) / BN, rb, nt);
      const int64_t row0 = (int64_t)rb * BM;
      if (SH && rb >= nbr) {  // a shared expert's row-block: tokens in order
        const int t0 = ((rb - nbr) % nbs) * BM + tid;
        if (tid < BM) {
          ms0 = t0 < Btok ? g.slots + t0 : -1;
          ms1 = tid + 1 < BM && t0 + 1 < Btok ? g.slots + t0 + 1 : -1;
        }
        if (tid == 0) me = g.E_loc + (rb - nbr) / nbs;
      } else {
        if (tid < BM) {
          ms0 = g.sorted_slots[row0 + tid];
          ms1 = tid + 1 < BM ? g.sorted_slots[row0 + tid + 1] : -1;
        }
        if (tid == 0) me = g.block_expert[rb];
      }
    };
    auto store_meta = [&](int j) __attribute__((always_inline)) {  // all threads; the caller's next barrier publishes it
      int* m = meta3 + (j % kMetaSlots) * META;
      if (tid < BM) {
        const bool v0 = ms0 >= 0 && ms0 < slot_end;
        const bool v1 = ms1 >= 0 && ms1 < slot_end;
        m[tid] = v0 ? ms0 : -1;
        if (v0 && !v1) m[BM] = tid + 1;    // last row of the leading run
        if (tid == 0 && !v0) m[BM] = 0;    // no row holds a slot
      }
      if (tid == 0) m[BM + 1] = me;
    };

    // ---- one stage: global -> registers, registers -> LDS ----
    // Operands are read with buffer loads: a 32-bit per-lane offset that stays
    // fixed for a tile, plus the stage's reduction offset as a scalar, so a stage
    // costs no address arithmetic.  A chunk that holds no operand (a padding row,
    // columns beyond K, a tile past the workgroup's last) gets an offset past the
    // buffer's range, and the hardware returns zeros for it without a memory
    // access: padding rows of A only reach output rows that are never stored,
    // zeros beyond K add nothing, and a missing tile is never computed.  Loads and LDS writes are branch-free, so the compiler can count
    // the loads in flight exactly and each stage waits only for its own data.
    // The load cursor (l_j, l_s) is the tile and stage of the next load; the
    // tile's row offsets and weight buffer are set once, when the cursor enters it.
    int l_j = 0, l_s = item_sb(0), l_se = item_se(0);
    bool l_new = true;  // the next load is the first of item l_j
    // A: the whole activation (x) or h buffer; byte offset of each chunk's row start
    const uint32_t a_bytes = PHASE == 1 ? (uint32_t)(g.slots / g.k) * (uint32_t)K * ASZ
                                        : (uint32_t)g.rows_max * (uint32_t)K * ASZ;
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(abase, a_bytes);
    uint32_t l_aoff[NA];
    // FP8 activation path: thread tid < BM * KB loads the A scale (x: per token;
    // h: per padded row) of tile row tid % BM, block tid / BM of each stage
    // (l_xsoff: that row's scale row, or kOob); threads tid < NMAT * NSB * KB load
    // the weight scales (l_wsbase: the tile's first scale of its first 128-row
    // block)
    const uint32_t a_rows = PHASE == 1 ? (uint32_t)(g.slots / g.k) : (uint32_t)g.rows_max;
    const __amdgpu_buffer_rsrc_t xs_rsrc =
        make_rsrc(g.xs, FP8A ? a_rows * (uint32_t)(K / 128) * 4u : 0u);
    uint32_t l_xsoff = kOob;
    int64_t l_wsbase = 0;
    // weights: per tile, a buffer from row n0 of the tile's expert matrix to its
    // end; each chunk's byte offset in it depends on the thread alone
    __amdgpu_buffer_rsrc_t l_b_rsrc[NMAT];
    uint32_t b_off[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = i * NT + tid;
      const int row = (q / GCB) % BN;
      b_off[i] = (uint32_t)(row * K + (q % GCB) * EPC_B) * WSZ;
    }
    int l_n0 = 0, l_e = 0;
    bool l_eok = false;
    auto enter_load_tile = [&](int j) __attribute__((always_inline)) {
      const int* m = meta3 + (j % kMetaSlots) * META;
      int rb, nt;
      tile_rc(item_tile(j), nb, (N + BN - 1) / BN, rb, nt);
      l_n0 = nt * BN;
      l_e = __builtin_amdgcn_readfirstlane(m[BM + 1]);
      l_eok = j < nitem && (unsigned)l_e < (unsigned)e_end;
      if (!l_eok) {
        l_e = 0;
        l_n0 = 0;
      }
      const int64_t wrow0 = ((int64_t)l_e * N + l_n0) * K;
      const uint32_t wbytes = l_eok ? (uint32_t)(N - l_n0) * (uint32_t)K * WSZ : 0u;
      l_b_rsrc[0] = make_rsrc(wmat0 + wrow0, wbytes);
      if constexpr (NMAT == 2) l_b_rsrc[1] = make_rsrc(wmat1 + wrow0, wbytes);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int q = i * NT + tid;
        const int row = q / GCA, c = q % GCA;
        const int sl = m[row];
        l_aoff[i] = kOob;
        if (l_eok && sl >= 0 && sl < slot_end) {
          // the host bounds every operand buffer below 2^31 bytes
          const int arow = PHASE == 1 ? (SH && sl >= g.slots ? sl - g.slots : sl / g.k) : rb * BM + row;
          l_aoff[i] = (uint32_t)(arow * K + c * EPC_A) * ASZ;
        }
      }
      if constexpr (FP8A) {
        const int sl = m[tid % BM];
        const int srow = PHASE == 1 ? (SH && sl >= g.slots ? sl - g.slots : sl / g.k) : rb * BM + tid % BM;
        l_xsoff = (l_eok && tid < BM * KB && sl >= 0 && sl < slot_end)
                      ? (uint32_t)srow * (uint32_t)(K / 128) * 4u + (uint32_t)(tid / BM) * 4u
                      : kOob;
        l_wsbase = l_eok ? ((int64_t)l_e * (N / 128) + l_n0 / 128) * (K / 128) : 0;
      }
    };
    auto load_stage = [&](Regs& R) __attribute__((always_inline)) {
      if (l_new) enter_load_tile(l_j);
      l_new = false;
      const int k0 = l_s * BK;
      const int kl = K - k0;  // reduction elements left from this stage on
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int kel = ((i * NT + tid) % GCA) * EPC_A;
        R.a[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, kel < kl ? l_aoff[i] : kOob, k0 * ASZ, 0));
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int q = i * NT + tid;
        const int mt = i * NT / (BN * GCB);  // one matrix per load instruction (tid < NT)
        const int kel = (q % GCB) * EPC_B;
        // non-temporal loads (cache policy nt) stream weights that no other tile reads
        R.b[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(l_b_rsrc[mt], kel < kl ? b_off[i] : kOob,
                                                         k0 * WSZ, STREAM ? kCacheNt : 0));
        if constexpr (FP8) {
          const int row = (q / GCB) % BN;
          const float* sm = mt == 0 ? smat0 : smat1;
          const bool ok = l_eok && kel < kl && l_n0 + row < N;  // rows past N have no scale
          R.s[i] = sm[ok ? ((int64_t)l_e * (N / 128) + (l_n0 + row) / 128) * (K / 128) + (k0 + kel) / 128 : 0];
        }
      }
      if constexpr (FP8A) {
        // scale blocks past K read as zero (x) or as a real scale (weights): the
        // operands there are zeros, so their products add nothing either way
        const int kb0 = k0 / 128;
        const bool xin = kb0 + tid / BM < K / 128;
        R.xs = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(xs_rsrc, xin ? l_xsoff : kOob, kb0 * 4, 0));
        // thread (mt * NSB + sb) * KB + kb: matrix mt, scale block sb of the tile's
        // columns, reduction block kb of the stage
        const float* sm = tid / (NSB * KB) == 0 ? smat0 : smat1;
        const bool wok = l_eok && tid < NMAT * NSB * KB && kb0 + tid % KB < K / 128 &&
                         l_n0 + ((tid / KB) % NSB) * 128 < N;  // no scale block past N
        R.ws = sm[wok ? l_wsbase + (int64_t)((tid / KB) % NSB) * (K / 128) + kb0 + tid % KB : 0];
      }
      if (++l_s == l_se) {  // past the last item the cursor runs on harmlessly
        ++l_j;
        l_s = item_sb(l_j);
        l_se = item_se(l_j);
        l_new = true;
      }
    };
    auto write_stage = [&](const Regs& R, uint8_t* buf) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int q = i * NT + tid;
        const int row = q / GCA, c = q % GCA;
        *(u32x4*)(buf + row * ROWB + ((c ^ tswz(row)) << 4)) = R.a[i];
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int q = i * NT + tid;
        const int c = q % GCB;
        const int row = BM + q / GCB;  // LDS row: matrices follow each other
        const int sw = tswz(row);
        uint8_t* rp = buf + row * ROWB;
        if constexpr (FP8) {
          u32x4 o0, o1;
          fp8x16_to_bf16(R.b[i], R.s[i], o0, o1);
          *(u32x4*)(rp + (((2 * c) ^ sw) << 4)) = o0;
          *(u32x4*)(rp + (((2 * c + 1) ^ sw) << 4)) = o1;
        } else {
          *(u32x4*)(rp + ((c ^ sw) << 4)) = R.b[i];
        }
      }
      if constexpr (FP8A) {  // the stage's scales; threads without one write the spare
        float* sc = (float*)(buf + ROWS * ROWB);
        sc[tid < BM * KB ? tid : SC_FLOATS - 1] = R.xs;
        sc[tid < NMAT * NSB * KB ? BM * KB + tid : SC_FLOATS - 1] = R.ws;
      }
    };

    // ---- MFMA over one stage ----
    f32x4 acc[NMAT][FM][FN];
    const int lr = lane & 15;   // row of the fragment
    const int lg = lane >> 4;   // k-group of 8 inside a 32-step
    // A fragment of 16 rows starting at row16 (a multiple of 16): lane row lr.  The
    // swizzle depends on row & 15 only, so a fragment's address is a per-lane
    // offset (frag_off) plus row16 * ROWB, which the fragment loops turn into
    // immediate offsets instead of one live address per fragment.
    auto frag_off = [&](int step, int half) __attribute__((always_inline)) {
      const int c0 = (FP8A || F32) ? step * 8 + 2 * lg + half : step * 4 + lg;
      return lr * ROWB + ((c0 ^ tswz(lr)) << 4);
    };
    auto read_frag = [&](const uint8_t* buf, int row16, int step, FragT& f) __attribute__((always_inline)) {
      const uint8_t* rp = buf + row16 * ROWB;
      if constexpr (FP8A) {  // 32 consecutive bytes of the step's 128-byte block
        f.lo = *(const u32x4*)(rp + frag_off(step, 0));
        f.hi = *(const u32x4*)(rp + frag_off(step, 1));
      } else if constexpr (F32) {
        f.lo = *(const f32x4*)(rp + frag_off(step, 0));
        f.hi = *(const f32x4*)(rp + frag_off(step, 1));
      } else {
        f.v = __builtin_bit_cast(bf16x8, *(const u32x4*)(rp + frag_off(step, 0)));
      }
    };
    // 16-row groups with no routed slot are skipped (their rows are never stored),
    // and a wave with none skips the stage.  A wave whose rows all hold a slot
    // takes a straight-line path (every fragment read and MFMA unconditional, so
    // reads and MFMAs interleave freely); only the last row-block of an expert
    // takes the guarded path.  Reduction steps beyond K need no guard: they were
    // loaded as zeros and add nothing.
    auto compute_full = [&](const uint8_t* buf) __attribute__((always_inline)) {
     const uint8_t* bufA = buf + wm * MW * ROWB;         // this wave's A rows
     const uint8_t* bufB = buf + (BM + wn * NW) * ROWB;  // its weight rows (matrix mt: + mt * BN rows)
     if constexpr (!FP8A && WIDE) {
      // wide class: the B fragments of a step stay in registers and the A
      // fragments are read one at a time, which keeps the 128 accumulators, two
      // register stages and the fragments within 256 registers
#pragma unroll
      for (int jj = 0; jj < KSTEPS / WK; ++jj) {
        const int step = jj * WK + wk;
        FragT fb[NMAT][FN];
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
          for (int j = 0; j < FN; ++j) read_frag(bufB, mt * BN + j * 16, step, fb[mt][j]);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          FragT fa;
          read_frag(bufA, i * 16, step, fa);
#pragma unroll
          for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int j = 0; j < FN; ++j) mma(acc[mt][i][j], fa, fb[mt][j]);
        }
      }
     } else if constexpr (!FP8A) {
#pragma unroll
      for (int jj = 0; jj < KSTEPS / WK; ++jj) {
        const int step = jj * WK + wk;
        FragT fa[FM];
        FragT fb[NMAT][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) read_frag(bufA, i * 16, step, fa[i]);
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
          for (int j = 0; j < FN; ++j) read_frag(bufB, mt * BN + j * 16, step, fb[mt][j]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int j = 0; j < FN; ++j) mma(acc[mt][i][j], fa[i], fb[mt][j]);
      }
     }
    };
    // FP8 activation path: each step is one 128-deep block; its sums are scaled by
    // the row's x scale times the tile's weight scale and added in fp32
    auto compute_f8 = [&](const uint8_t* buf, int nvalid) __attribute__((always_inline)) {
     const uint8_t* bufA = buf + wm * MW * ROWB;         // this wave's A rows
     const uint8_t* bufB = buf + (BM + wn * NW) * ROWB;  // its weight rows (matrix mt: + mt * BN rows)
     if constexpr (FP8A) {
      if (wm * MW >= nvalid) return;
      const bool full = wm * MW + MW <= nvalid;
      const float* sc = (const float*)(buf + ROWS * ROWB);
#pragma unroll
      for (int jj = 0; jj < KSTEPS / WK; ++jj) {
        const int step = jj * WK + wk;
        FragT fb[NMAT][FN];
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
          for (int j = 0; j < FN; ++j) read_frag(bufB, mt * BN + j * 16, step, fb[mt][j]);
        float wsv[NMAT];
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) wsv[mt] = sc[BM * KB + (mt * NSB + (wn * NW) / 128) * KB + step];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          if (!full && wm * MW + i * 16 >= nvalid) continue;
          FragT fa;
          read_frag(bufA, i * 16, step, fa);
          // x scales of this lane's output rows 4 * (lane / 16) + c
          const f32x4 xsv = *(const f32x4*)(sc + step * BM + wm * MW + i * 16 + 4 * lg);
#pragma unroll
          for (int mt = 0; mt < NMAT; ++mt) {
            f32x4 s4;
#pragma unroll
            for (int c = 0; c < 4; ++c) s4[c] = xsv[c] * wsv[mt];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const f32x4 t = mma_fp8_block(fa, fb[mt][j]);
#pragma unroll
              for (int c = 0; c < 4; ++c) acc[mt][i][j][c] = __builtin_fmaf(t[c], s4[c], acc[mt][i][j][c]);
            }
          }
        }
      }
     }
    };
    auto compute_stage = [&](const uint8_t* buf, int nvalid) __attribute__((always_inline)) {
     const uint8_t* bufA = buf + wm * MW * ROWB;         // this wave's A rows
     const uint8_t* bufB = buf + (BM + wn * NW) * ROWB;  // its weight rows (matrix mt: + mt * BN rows)
     if constexpr (FP8A) {
      compute_f8(buf, nvalid);
     } else {
      if (wm * MW >= nvalid) return;
      if (wm * MW + MW <= nvalid) {
        compute_full(buf);
        return;
      }
      if constexpr (WIDE) {  // as compute_full, one A fragment at a time
#pragma unroll
        for (int jj = 0; jj < KSTEPS / WK; ++jj) {
          const int step = jj * WK + wk;
          FragT fb[NMAT][FN];
#pragma unroll
          for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int j = 0; j < FN; ++j) read_frag(bufB, mt * BN + j * 16, step, fb[mt][j]);
#pragma unroll
          for (int i = 0; i < FM; ++i)
            if (wm * MW + i * 16 < nvalid) {
              FragT fa;
              read_frag(bufA, i * 16, step, fa);
#pragma unroll
              for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
                for (int j = 0; j < FN; ++j) mma(acc[mt][i][j], fa, fb[mt][j]);
            }
        }
        return;
      }
#pragma unroll
      for (int jj = 0; jj < KSTEPS / WK; ++jj) {
        const int step = jj * WK + wk;
        FragT fa[FM];
        FragT fb[NMAT][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          if (wm * MW + i * 16 < nvalid) read_frag(bufA, i * 16, step, fa[i]);
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
          for (int j = 0; j < FN; ++j) read_frag(bufB, mt * BN + j * 16, step, fb[mt][j]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
          if (wm * MW + i * 16 < nvalid) {
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
              for (int j = 0; j < FN; ++j) mma(acc[mt][i][j], fa[i], fb[mt][j]);
          }
      }
     }
    };

    // ---- epilogue of item j: K-split reduction, then the tile's stores, or the
    // piece's fp32 sums to its slot of g.part ----
    auto epilogue = [&](int j, uint8_t* red_area, bool whole) __attribute__((always_inline)) {
      const int* m = meta3 + (j % kMetaSlots) * META;
      int rb, nt;
      tile_rc(item_tile(j), nb, (N + BN - 1) / BN, rb, nt);
      const int64_t row0 = (int64_t)rb * BM;
      const int n0 = nt * BN;
      if ((unsigned)m[BM + 1] >= (unsigned)e_end) return;  // uniform: no such tile
      if constexpr (WK > 1) {
        // waves wk > 0 hand their sums to wave wk = 0 through the LDS buffer just
        // computed on (the barrier first lets every wave finish reading it)
        float* red = (float*)red_area;
        constexpr int PER = NMAT * FM * FN * 4 * 64;
        const int rslot = (wm * WN + wn) * (WK - 1);
        __syncthreads();
        if (wk > 0) {
          float* dst = red + (rslot + wk - 1) * PER;
#pragma unroll
          for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int jn = 0; jn < FN; ++jn)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                  dst[(((mt * FM + i) * FN + jn) * 4 + c) * 64 + lane] = acc[mt][i][jn][c];
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll
          for (int qq = 0; qq < WK - 1; ++qq) {
            const float* src = red + (rslot + qq) * PER;
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
              for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int jn = 0; jn < FN; ++jn)
#pragma unroll
                  for (int c = 0; c < 4; ++c)
                    acc[mt][i][jn][c] += src[(((mt * FM + i) * FN + jn) * 4 + c) * 64 + lane];
          }
        }
      }
      if (wk == 0) {
        if (whole) {
          store_acc(g, acc, m, row0, n0, wm, wn, lane);
        } else {
          // piece slot j - Fw of this workgroup; 16 bytes per lane, wave-contiguous
          float* dst = g.part + ((int64_t)slot * 2 + (j - Fw)) * PIECE + (wm * WN + wn) * NFRAG * 256;
#pragma unroll
          for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int jn = 0; jn < FN; ++jn)
                *(f32x4*)(dst + (((mt * FM + i) * FN + jn) * 64 + lane) * 4) = acc[mt][i][jn];
        }
      }
    };

    // ---- the pipeline: RS register stages ahead, two LDS buffers ----
    // Items whose first stage is among the first RS + 1 are described before the
    // loop; a later item j' is fetched at the step whose load is the last stage
    // before it and stored at the next step, before that step's barrier and the
    // load of its first stage.
    Regs R[RS];
    for (int j = 0; j < nitem; ++j) {
      const int start = j <= Fw ? j * nst : Fw * nst + item_se(Fw) - sb0;  // first stage of item j
      if (start > RS) break;
      fetch_meta(j);
      store_meta(j);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < RS; ++u)
      if (u < nv) load_stage(R[u]);
    int c_j = 0, c_s = item_sb(0), c_sb = c_s, c_se = item_se(0);  // item and stage being computed
    // one pipeline step: stage v from registers Ru to LDS, the load of stage
    // v + RS into Ru, the MFMAs of stage v
    auto step = [&](const int v, Regs& Ru) __attribute__((always_inline)) {
          const int* m = meta3 + (c_j % kMetaSlots) * META;
          uint8_t* buf = (v & 1) ? lds1 : lds0;
          write_stage(Ru, buf);
          const bool more = v + RS < nv;  // a real load follows this step
          if (more && l_new && v >= 1) store_meta(l_j);
          if (v + RS + 1 < nv && l_s == l_se - 1) fetch_meta(l_j + 1);
          __syncthreads();
          load_stage(Ru);  // past the last stage its offsets are out of range
          if (c_s == c_sb) {
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
              for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int jn = 0; jn < FN; ++jn) acc[mt][i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          if ((unsigned)m[BM + 1] < (unsigned)e_end) compute_stage(buf, m[BM]);
          if (c_s == c_se - 1) epilogue(c_j, buf, c_sb == 0 && c_se == nst);
          if (++c_s == c_se) {
            ++c_j;
            c_s = c_sb = item_sb(c_j);
            c_se = item_se(c_j);
          }
    };
    // The compiler's wait before each stage's LDS write also covers the younger
    // register stage's loads (the steps are conditional), so about one stage of
    // loads is in flight at that point.  Loops with exact waits (two stages in
    // flight) measured slower on the cached large-tile configuration, and no
    // faster elsewhere.
    for (int v0 = 0; v0 < nv; v0 += RS) {
#pragma unroll
      for (int u = 0; u < RS; ++u)
        if (v0 + u < nv) step(v0 + u, R[u]);
    }
  }

  // ---------------------------------------------------------------------------
  // The wide class's bf16 tiles with direct global -> LDS loads.  Each stage's A
  // rows and weight rows go from HBM (or L2) straight into one of ND LDS stage
  // buffers with the buffer-load LDS form of gfx950, ND stages ahead of the
  // MFMAs and with no register staging, so the loads in flight are bounded by LDS
  // (ND x 32 KiB) instead of by registers.  Four waves, one per SIMD, each own a
  // 128 x 128 block of the tile: its 256 fp32 sums per lane stay in the
  // accumulation registers for the whole reduction, and the fragments of the next
  // stage are read from LDS into a second register set while the MFMAs of this
  // stage run, so one wave per SIMD keeps its matrix unit fed.  Loads past the
  // last stage (and of rows that hold no slot) use an offset past the buffer's
  // range: no memory is read.
  static constexpr int kDmaInstr = ROWS * C / NT;  // 16-byte loads per thread per stage
  // s_waitcnt vmcnt(N_) lgkmcnt(0), then s_barrier, as builtins: the compiler
  // then knows which of its loads and LDS reads are complete (an inline-asm wait
  // is opaque to it, and it would add waits of its own after it).  gfx9 encoding:
  // vmcnt in bits 3:0 and 15:14, expcnt (7: none) in 6:4, lgkmcnt in 11:8.
  template <int N_>
  __device__ __forceinline__ static void wait_vm_bar() {
    static_assert(N_ >= 0 && N_ < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N_ & 15) | ((N_ >> 4) << 14) | (7 << 4));
    __builtin_amdgcn_s_barrier();
  }

  // ---- the wide class's tile order and tail split ----
  // pexp[e] (e = 0..e_end) = the first row-block of local expert e, from a pass
  // over the block experts: the experts in (expert of block b - 1, expert of
  // block b] start at block b (each entry written by exactly one thread).  Tile t
  // then lies in the run of row-blocks [pexp[e], pexp[e + 1]) that holds block
  // t / ncol, and the run's tiles go column tile by column tile, its row-blocks
  // fastest: the G / 8 consecutive slots that share an XCD then hold every
  // row-block of a few weight tiles, and that L2 serves each weight slice to all
  // of its row-blocks.  Block experts out of range or not in ascending order (not
  // what the alignment step writes) fall back to tile_rc's order: the return
  // value is then nonzero.  Every thread of the workgroup calls this (barrier).
  template <bool SH>
  __device__ __forceinline__ static int expert_runs(const FfnArgs& g, int* pexp, int nb, int nbr,
                                                   int nbs, int e_end) {
    auto bexp = [&](int b) __attribute__((always_inline)) {
      return SH && b >= nbr ? g.E_loc + (b - nbr) / nbs : g.block_expert[b];
    };
    int bad = e_end > kRunTable - 1;
    if (!bad) {
      for (int b = threadIdx.x; b <= nb; b += NT) {
        const int e1 = b < nb ? bexp(b) : e_end;
        const int e0 = b > 0 ? bexp(b - 1) : -1;
        if ((b < nb && (unsigned)e1 >= (unsigned)e_end) || e1 < e0) {
          bad = 1;
        } else {
          for (int e = e0 + 1 > 0 ? e0 + 1 : 0; e <= e1; ++e) pexp[e] = b;
        }
      }
    }
    return __syncthreads_or(bad);
  }
  __device__ __forceinline__ static void tile_map(const int* pexp, int bad, int e_end, int t, int nb,
                                                  int ncol, int& rb, int& nt) {
    if (bad) {
      tile_rc(t, nb, ncol, rb, nt);
      return;
    }
    const int b = t / ncol;
    int lo = 0, hi = e_end;  // pexp[lo] <= b < pexp[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pexp[mid] <= b)
        lo = mid;
      else
        hi = mid;
    }
    const int s0 = pexp[lo], n = pexp[lo + 1] - s0;
    const int local = t - s0 * ncol;
    nt = local / n;
    rb = s0 + (local - nt * n);
  }
  // Tail split of the wide class's down phase (hybrid Stream-K): after F >= 1 full
  // rounds, a last round of r <= G / 2 tiles would leave most of the grid idle
  // for a whole tile of the longest reduction in the layer.  Each tail tile is
  // then cut into P pieces of whole four-stage groups, one piece per workgroup
  // (workgroup slot w < r * P takes piece w % P of tail tile w / P), so that
  // every stage loop still starts on buffer 0 and each workgroup leaves at most
  // one partial tile.  Pieces hold at least two groups (the next item's metadata
  // is fetched five stages before its first load).  Returns P, or 0: no split.
  __device__ __forceinline__ static int wide_pieces(int r, int G, int F, int nst) {
    if (PHASE != 2 || F < 1 || r <= 0 || 2 * r > G || (int64_t)G * PIECE > kPartBytes / 4) return 0;
    int P = G / r;
    if (P > nst / 8) P = nst / 8;
    return P >= 2 ? P : 0;
  }

  template <bool SH, int ND>
  __device__ __forceinline__ static void run_dma(const FfnArgs& g, uint8_t* b0, uint8_t* b1,
                                                 uint8_t* b2, uint8_t* b3, int* meta3, int* pexp,
                                                 uint8_t* ostage, int nb, int nbr, int slot, int G) {
    static_assert(WKIND == W_BF16 && WIDE && WM == 2 && WN == 2 && WK == 1 && KSTEPS == 1 && C == 4,
                  "the direct-load pipeline serves the wide class's bf16 tiles");
    static_assert(ND == 4, "four stage buffers");
    static_assert(NT == BM && ROWS == 2 * NT && NMAT * BN == BM && kDmaInstr == 8,
                  "load instruction i covers stage rows 64 i .. 64 i + 63: A rows, then weight rows");
    static_assert(FM == 8 && NMAT * FN == 8, "a wave owns 8 x 8 accumulator blocks");
    const int N = PHASE == 1 ? g.I : g.H;
    const int K = PHASE == 1 ? g.H : g.I;
    const int Btok = g.slots / g.k;
    const int nbs = SH ? (Btok + BM - 1) / BM : 1;
    const int slot_end = SH ? g.slots + Btok : g.slots;
    const int e_end = SH ? g.E_loc + g.n_shared : g.E_loc;
    const int ncol = (N + BN - 1) / BN;
    const int total = nb * ncol;
    const int nst = K / BK;  // the caller checks K % (ND * BK) == 0 and nst >= ND
    const int F = total / G;
    const int r = total - F * G;
    // work items: whole tiles slot, slot + G, ..., then at most one tail piece
    const int P = wide_pieces(r, G, F, nst);
    const int nwhole = F + (P == 0 && slot < r ? 1 : 0);
    const bool has_piece = P > 0 && slot < r * P;
    const int nit = nwhole + (has_piece ? 1 : 0);
    if (nit == 0) return;
    const int ngr = nst / ND;
    const int pq = has_piece ? slot % P : 0;
    const int psb = has_piece ? ND * (pq * ngr / P) : 0;
    const int pse = has_piece ? ND * ((pq + 1) * ngr / P) : nst;
    auto item_tile = [&](int j) __attribute__((always_inline)) {
      return j < nwhole ? slot + j * G : F * G + (has_piece ? slot / P : 0);
    };
    auto item_sb = [&](int j) __attribute__((always_inline)) { return j == nwhole ? psb : 0; };
    auto item_se = [&](int j) __attribute__((always_inline)) { return j == nwhole ? pse : nst; };
    const int tid = threadIdx.x;
    // wave coordinates in scalar registers: every row test below is then a scalar
    // branch, not an exec mask around each group of MFMAs
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wn = wave % WN;
    const int wm = wave / WN;
    const Act* abase = (const Act*)(PHASE == 1 ? g.x : g.h);
    const Wt* wmat0 = (const Wt*)(PHASE == 1 ? g.w1 : g.w2);
    const Wt* wmat1 = (const Wt*)(PHASE == 1 ? g.w3 : g.w2);

    // ---- tile order: expert-major, row-block fastest (expert_runs) ----
    const int bad = expert_runs<SH>(g, pexp, nb, nbr, nbs, e_end);

    // ---- tile metadata (as run_all: a ring of kMetaSlots slots in LDS) ----
    int ms0 = -1, ms1 = -1, me = -1, m_rb = 0, m_nt = 0;
    auto fetch_meta = [&](int j) __attribute__((always_inline)) {
      int rb, nt;
      tile_map(pexp, bad, e_end, item_tile(j), nb, ncol, rb, nt);
      m_rb = rb;
      m_nt = nt;
      const int64_t row0 = (int64_t)rb * BM;
      if (SH && rb >= nbr) {
        const int t0 = ((rb - nbr) % nbs) * BM + tid;
        ms0 = t0 < Btok ? g.slots + t0 : -1;
        ms1 = tid + 1 < BM && t0 + 1 < Btok ? g.slots + t0 + 1 : -1;
        if (tid == 0) me = g.E_loc + (rb - nbr) / nbs;
      } else {
        ms0 = g.sorted_slots[row0 + tid];
        ms1 = tid + 1 < BM ? g.sorted_slots[row0 + tid + 1] : -1;
        if (tid == 0) me = g.block_expert[rb];
      }
    };
    auto store_meta = [&](int j) __attribute__((always_inline)) {
      int* m = meta3 + (j % kMetaSlots) * META;
      const bool v0 = ms0 >= 0 && ms0 < slot_end;
      const bool v1 = ms1 >= 0 && ms1 < slot_end;
      m[tid] = v0 ? ms0 : -1;
      if (v0 && !v1) m[BM] = tid + 1;
      if (tid == 0 && !v0) m[BM] = 0;
      if (tid == 0) {
        m[BM + 1] = me;
        m[BM + 2] = m_rb;
        m[BM + 3] = m_nt;
      }
    };

    // ---- the loads of one stage ----
    // Load instruction i of thread tid fills LDS chunk i * NT + tid of the stage
    // buffer: row 64 i + tid / 4, physical chunk tid % 4, which holds logical
    // chunk (tid % 4) ^ swz(row) (the swizzle of the fragment reads).
    // Instructions 0-3 take A rows 0-255, 4-7 weight rows 0-255 (gate/up: W1 rows
    // n0 .. n0 + 127, then the same rows of W3; down: W2).
    const int c_log = (tid & 3) ^ ((tid >> 3) & 3);  // swz<4>(64 i + tid / 4)
    // gate/up: x rows through one descriptor; down: the row-block's blocks of h
    // (hblock_offset), a descriptor per item
    __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(abase, PHASE == 1 ? (uint32_t)Btok * (uint32_t)K * ASZ : 0u);
    uint32_t l_aoff[4] = {kOob, kOob, kOob, kOob};
    // Weights from the packed copy (moe_pack_wide): each stage of a tile is one
    // 256-row block of 64-byte rows (gate/up: W1's 128 rows, then W3's), so
    // instruction i reads block rows 64 i .. 64 i + 63; else from W1/W3/W2 rows.
    const bool pk = g.wpk != nullptr;
    uint32_t l_boff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = pk || NMAT == 1 ? i * 64 + (tid >> 2) : (i & 1) * 64 + (tid >> 2);
      l_boff[i] = (uint32_t)rr * (pk ? 64u : (uint32_t)K * WSZ) + c_log * 16;
    }
    static_assert(ROWB == 64 && BM == 256 && NMAT * BN == 256, "packed blocks are 256 rows x 64 bytes");
    constexpr uint32_t kPkBlock = 256 * 64;  // bytes of one packed stage
    // this phase's region of the packed copy: gate/up first, then down
    const int64_t pk_region = PHASE == 1 ? 0
                                         : (int64_t)(g.E_loc + g.n_shared) * ((g.I + 127) / 128) *
                                               (g.H / 32) * kPkBlock;
    __amdgpu_buffer_rsrc_t l_b_rsrc[2];
    int l_j = 0, l_s = item_sb(0), l_se = item_se(0);
    bool l_new = true;
    auto enter_load_tile = [&](int j) __attribute__((always_inline)) {
      const int* m = meta3 + (j % kMetaSlots) * META;
      const int rb = __builtin_amdgcn_readfirstlane(m[BM + 2]);
      const int nt = __builtin_amdgcn_readfirstlane(m[BM + 3]);
      int e = __builtin_amdgcn_readfirstlane(m[BM + 1]);
      int n0 = nt * BN;
      const bool eok = j < nit && (unsigned)e < (unsigned)e_end;
      if (!eok) {
        e = 0;
        n0 = 0;
      }
      if (pk) {
        // the tile's nst consecutive blocks; rows past N are zeros in the copy
        const uint8_t* tb = g.wpk + pk_region + ((int64_t)e * ncol + (eok ? nt : 0)) * nst * kPkBlock;
        l_b_rsrc[0] = make_rsrc(tb, eok ? (uint32_t)nst * kPkBlock : 0u);
        l_b_rsrc[1] = l_b_rsrc[0];
      } else {
        const int64_t wrow0 = ((int64_t)e * N + n0) * K;
        const uint32_t wbytes = eok ? (uint32_t)(N - n0) * (uint32_t)K * WSZ : 0u;
        l_b_rsrc[0] = make_rsrc(wmat0 + wrow0, wbytes);
        l_b_rsrc[1] = make_rsrc(wmat1 + wrow0, wbytes);
      }
      if constexpr (PHASE == 2)
        a_rsrc = make_rsrc((const uint8_t*)g.h + hblock_offset(g, eok ? rb : 0, 0),
                           eok ? (uint32_t)nst * 256u * 64u : 0u);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = i * 64 + (tid >> 2);
        const int sl = m[row];
        l_aoff[i] = kOob;
        if (eok && sl >= 0 && sl < slot_end) {
          if constexpr (PHASE == 1) {
            const int arow = SH && sl >= g.slots ? sl - g.slots : sl / g.k;
            l_aoff[i] = (uint32_t)(arow * K + c_log * 8) * ASZ;
          } else {
            l_aoff[i] = (uint32_t)(row * 64 + c_log * 16);
          }
        }
      }
    };
    // A stage's loads in three parts, so that a step can spread its load
    // instructions among its MFMAs: issue_begin (the item's offsets when a new
    // item starts), issue_one(buf, i) for i = 0 .. kDmaInstr - 1, issue_end.
    int l_soff = 0, l_bsoff = 0, l_woff = 0;
    auto issue_begin = [&]() __attribute__((always_inline)) {
      if (l_new) enter_load_tile(l_j);
      l_new = false;
      l_soff = PHASE == 1 ? l_s * BK * ASZ : l_s * 256 * 64;  // x rows; blocks of h
      l_bsoff = pk ? l_s * (int)kPkBlock : l_s * BK * WSZ;
      // this wave's LDS offset, opaque to the compiler at every step: each load's
      // destination is then one scalar add (hoisted, the 32 destinations of the
      // four buffers were kept in scalar registers, which spilled)
      l_woff = wave * 64 * 16;
      asm volatile("" : "+s"(l_woff));
    };
    auto issue_one = [&](uint8_t* buf, int i) __attribute__((always_inline)) {
      typedef __attribute__((address_space(3))) void lds_void;
      lds_void* dst = (lds_void*)(buf + i * NT * 16 + l_woff);
      if (i < 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, dst, 16, l_aoff[i], l_soff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(l_b_rsrc[NMAT == 2 ? (i - 4) >> 1 : 0], dst, 16,
                                                 l_boff[i - 4], l_bsoff, 0, 0);
    };
    auto issue_end = [&]() __attribute__((always_inline)) {
      if (++l_s == l_se) {  // past the last item the offsets are out of range
        ++l_j;
        l_s = item_sb(l_j);
        l_se = item_se(l_j);
        l_new = true;
      }
    };
    auto issue = [&](uint8_t* buf) __attribute__((always_inline)) {
      issue_begin();
#pragma unroll
      for (int i = 0; i < kDmaInstr; ++i) issue_one(buf, i);
      issue_end();
    };

    // ---- accumulators, fragments and MFMAs ----
    // The MFMAs are written as inline asm with the accumulator tied in place
    // ("+a"): the sums then stay in the same accumulation registers from stage to
    // stage (with the builtin, the register allocator rotated them through copies).
    // The compiler does not see these as MFMAs, so it inserts no hazard padding
    // for them: after an item's last MFMAs, an explicit s_nop of 19 wait states
    // covers the longest MFMA-result-to-read requirement before any read of the
    // sums; the zeroing before the first MFMAs of an item is separated from them
    // by the stage loop's barrier, loads and LDS reads.  Fragment operands come
    // from LDS reads, which the compiler's own counter waits cover.
    f32x4 acc[NMAT][FM][FN];
    const int lr = lane & 15, lg = lane >> 4;
    const int foff = lr * ROWB + ((lg ^ swz<C>(lr)) << 4);
    auto buf_of = [&](int u) __attribute__((always_inline)) {
      return u == 0 ? b0 : (u == 1 ? b1 : (u == 2 ? b2 : b3));
    };
    bf16x8 fa0[FM], fb0[NMAT * FN], fa1[FM], fb1[NMAT * FN];
    // fragment k of a stage: k < NMAT FN the weight fragments, then the A ones
    auto read_one = [&](const uint8_t* buf, int k, bf16x8(&fa)[FM], bf16x8(&fb)[NMAT * FN])
        __attribute__((always_inline)) {
      if (k < NMAT * FN)
        fb[k] = *(const bf16x8*)(buf + (BM + wn * NW + (k / FN) * BN + (k % FN) * 16) * ROWB + foff);
      else
        fa[k - NMAT * FN] = *(const bf16x8*)(buf + (wm * MW + (k - NMAT * FN) * 16) * ROWB + foff);
    };
    auto read_frags = [&](const uint8_t* buf, bf16x8(&fa)[FM], bf16x8(&fb)[NMAT * FN])
        __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < NMAT * FN + FM; ++k) read_one(buf, k, fa, fb);
    };
    // MFMAs q0 .. q1 - 1 of A fragment row i (weight fragment q of each)
    auto mfmas = [&](int i, int q0, int q1, const bf16x8(&fa)[FM], const bf16x8(&fb)[NMAT * FN])
        __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < NMAT * FN; ++q)
        if (q >= q0 && q < q1)
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                       : "+a"(acc[q / FN][i][q % FN])
                       : "v"(fa[i]), "v"(fb[q]));
    };
    // One step's work after its barrier, in FM groups, each: the MFMAs of one A
    // fragment row of this stage, with two fragment reads of the next stage and
    // one load instruction of the stage ND ahead spread among them (read, two
    // MFMAs, read, two MFMAs, load, four MFMAs).  A wave per SIMD issues
    // everything itself, so spreading the loads and LDS reads among the MFMAs
    // keeps the matrix unit busy while they queue: issued all before the MFMAs,
    // they left it idle for about half of each step; among them, placed as here,
    // measured fastest of the orders tried.  Memory operations keep their program
    // order around the volatile MFMA asm.
    static_assert(FM == kDmaInstr && 2 * FM == NMAT * FN + FM && NMAT * FN == 8,
                  "one load, two reads and eight MFMAs per group");
    auto groups = [&](uint8_t* dbuf, const uint8_t* rbuf, bf16x8(&nfa)[FM], bf16x8(&nfb)[NMAT * FN],
                      const bf16x8(&cfa)[FM], const bf16x8(&cfb)[NMAT * FN])
        __attribute__((always_inline)) {
#pragma unroll
      for (int gi = 0; gi < FM; ++gi) {
        // fragment reads front-loaded: three in each of groups 0-3, two in 4-5
        constexpr int kR[FM + 1] = {0, 3, 6, 9, 12, 14, 16, 16, 16};
        const int r0 = kR[gi], nr = kR[gi + 1] - kR[gi];
        if (nr > 0) read_one(rbuf, r0, nfa, nfb);
        mfmas(gi, 0, 2, cfa, cfb);
        if (nr > 1) read_one(rbuf, r0 + 1, nfa, nfb);
        mfmas(gi, 2, 4, cfa, cfb);
        if (nr > 2) read_one(rbuf, r0 + 2, nfa, nfb);
        mfmas(gi, 4, 6, cfa, cfb);
        issue_one(dbuf, gi);
        mfmas(gi, 6, 8, cfa, cfb);
      }
    };

    // ---- the pipeline ----
    // Tile loop around a stage loop unrolled by ND, the tile's stores after it: the
    // accumulators live across the stage loop only.  Every item has a multiple of
    // ND stages and starts at a multiple of ND (the caller checks nst % ND == 0),
    // so stage s of any item sits in buffer s % ND, its fragments in register set
    // s % 2, and each unrolled step names both at compile time.  Step s: wait until
    // this wave's loads of stage s + 1 are in LDS and its LDS reads of stage s are
    // in registers, then a barrier (every wave's loads of stage s + 1 are visible,
    // and every wave holds stage s's fragments, so stage s's buffer is free); issue
    // the loads of stage s + ND into that buffer, read stage s + 1's fragments
    // (the next item's first stage after an item's last), and run stage s's MFMAs.
    // Each stage's loads so have ND - 1 steps to land.  The loads run ND stages
    // ahead across items: item j + 1's metadata is fetched at stage se - ND - 1
    // of item j and stored at stage se - ND, before the barrier of the step that
    // issues its first loads (an item of only ND stages fetches it at that step
    // too).  Every wave runs all its MFMAs, also on rows with no slot (loaded out
    // of range as zeros; their sums are never stored): the barrier paces a step
    // by its slowest wave, so skipping them would save no time, and the test
    // between MFMAs cost about a tenth of each step.
    fetch_meta(0);
    store_meta(0);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < ND; ++u) issue(buf_of(u));
    wait_vm_bar<(ND - 1) * kDmaInstr>();  // stage 0 in LDS
    read_frags(b0, fa0, fb0);
    for (int j = 0; j < nit; ++j) {
      const int* m = meta3 + (j % kMetaSlots) * META;
      const int len = item_se(j) - item_sb(j);
      const bool live = (unsigned)__builtin_amdgcn_readfirstlane(m[BM + 1]) < (unsigned)e_end;
      const bool more = j + 1 < nit;
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int jn = 0; jn < FN; ++jn) acc[mt][i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};
      // step c of the item: its stage sb + c (the loop counts from the item's
      // start, so that every item runs the same loop)
      auto step = [&](int c0, auto U) __attribute__((always_inline)) {
        constexpr int u = decltype(U)::value;
        const int c = c0 + u;
        // (an item of only ND stages fetches at its first step, just before storing)
        if (more && c == (len - ND - 1 > 0 ? len - ND - 1 : 0)) fetch_meta(j + 1);
        if (more && c == len - ND) store_meta(j + 1);
        // stage s + 1 is the oldest but ND - 2 stages of this wave's loads
        wait_vm_bar<(ND - 2) * kDmaInstr>();
        issue_begin();
        if constexpr ((u & 1) == 0)
          groups(buf_of(u), buf_of((u + 1) % ND), fa1, fb1, fa0, fb0);
        else
          groups(buf_of(u), buf_of((u + 1) % ND), fa0, fb0, fa1, fb1);
        issue_end();
        // after the item's last MFMAs, the padding before any read of the sums:
        // inside the loop, so every read after it (wherever the compiler places
        // it) follows in execution order
        if constexpr (u == ND - 1)
          if (c0 + ND >= len) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2" ::: "memory");
      };
      // every item has at least ND stages: a loop with no path around it
      int c0 = 0;
      do {
        step(c0, std::integral_constant<int, 0>{});
        step(c0, std::integral_constant<int, 1>{});
        step(c0, std::integral_constant<int, 2>{});
        step(c0, std::integral_constant<int, 3>{});
        c0 += ND;
      } while (c0 < len);
      if (live) {
        if (j < nwhole) {
          const int rb = __builtin_amdgcn_readfirstlane(m[BM + 2]);
          const int nt = __builtin_amdgcn_readfirstlane(m[BM + 3]);
          store_staged(g, acc, m, (int64_t)rb * BM, nt * BN, wm, wn, lane, ostage + wave * OSTAGE);
        } else {
          // this workgroup's piece: its fp32 sums in MFMA fragment order, 16 bytes
          // per lane, wave-contiguous (wide_fixup adds the pieces).  Buffer
          // stores with the fragment's offset as a constant: no per-fragment
          // address is formed (or kept live across the stage loop)
          const __amdgpu_buffer_rsrc_t prs =
              make_rsrc(g.part + (int64_t)slot * PIECE + wave * NFRAG * 256, NFRAG * 256 * 4);
#pragma unroll
          for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int jn = 0; jn < FN; ++jn)
              {
                const f32x4& a = acc[mt][i][jn];
                const f32x4 v = {acc_read(a, 0), acc_read(a, 1), acc_read(a, 2), acc_read(a, 3)};
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), prs, lane * 16,
                                                       ((mt * FM + i) * FN + jn) * 1024, 0);
              }
        }
      }
    }
    // every load of this workgroup has landed before it exits (the last steps'
    // loads were out of range, so this costs nothing)
    __builtin_amdgcn_s_waitcnt(0);
  }

  // The fix-up of the wide class's split tail tile tq (see wide_pieces): adds its
  // P pieces in reduction order (piece q, workgroup slot tq * P + q, holds stages
  // [4 (q ngr / P), 4 ((q + 1) ngr / P)) ) and stores the tile.  Two workgroups
  // share a tile, one per half of each wave's rows (half = 0, 1); each wave adds
  // its fragment region two 16-row groups at a time, with all of a piece's loads
  // for those rows in flight together.
  template <bool SH>
  __device__ __forceinline__ static void wide_fixup(const FfnArgs& g, int* meta, int* pexp, int nb,
                                                    int nbr, int G, int tq, int half) {
    const int N = PHASE == 1 ? g.I : g.H;
    const int K = PHASE == 1 ? g.H : g.I;
    const int ncol = (N + BN - 1) / BN;
    const int total = nb * ncol;
    const int nst = K / BK;
    const int F = total / G;
    const int r = total - F * G;
    const int P = wide_pieces(r, G, F, nst);
    if (P == 0 || tq >= r) return;  // uniform over the workgroup
    const int Btok = g.slots / g.k;
    const int nbs = SH ? (Btok + BM - 1) / BM : 1;
    const int slot_end = SH ? g.slots + Btok : g.slots;
    const int e_end = SH ? g.E_loc + g.n_shared : g.E_loc;
    const int bad = expert_runs<SH>(g, pexp, nb, nbr, nbs, e_end);
    int rb, nt;
    tile_map(pexp, bad, e_end, F * G + tq, nb, ncol, rb, nt);
    const int e = SH && rb >= nbr ? g.E_loc + (rb - nbr) / nbs : g.block_expert[rb];
    if ((unsigned)e >= (unsigned)e_end) return;  // uniform: the pieces were not stored
    const int tid = threadIdx.x;
    for (int row = tid; row < BM; row += NT) {
      int sl;
      if (SH && rb >= nbr) {
        const int t0 = ((rb - nbr) % nbs) * BM + row;
        sl = t0 < Btok ? g.slots + t0 : -1;
      } else {
        sl = g.sorted_slots[(int64_t)rb * BM + row];
      }
      meta[row] = sl >= 0 && sl < slot_end ? sl : -1;
    }
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wn = wave % WN, wm = wave / WN;
    constexpr int FG = 2;
    static_assert(FM % (2 * FG) == 0, "each half is whole groups of FG row groups");
#pragma unroll 1
    for (int i0 = half * (FM / 2); i0 < (half + 1) * (FM / 2); i0 += FG) {
      f32x4 acc[NMAT][FG][FN];
      for (int q = 0; q < P; ++q) {
        const float* src = g.part + (int64_t)(tq * P + q) * PIECE + wave * NFRAG * 256;
        f32x4 v[NMAT][FG][FN];
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
          for (int i = 0; i < FG; ++i)
#pragma unroll
            for (int jn = 0; jn < FN; ++jn)
              v[mt][i][jn] = *(const f32x4*)(src + (((mt * FM + i0 + i) * FN + jn) * 64 + lane) * 4);
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
          for (int i = 0; i < FG; ++i)
#pragma unroll
            for (int jn = 0; jn < FN; ++jn)
              acc[mt][i][jn] = q == 0 ? v[mt][i][jn] : acc[mt][i][jn] + v[mt][i][jn];
      }
      store_rows<FG>(g, acc, meta, (int64_t)rb * BM, nt * BN, wm, wn, lane, i0);
    }
  }

  // The fix-up of tail tile tq (the tile F * G + tq of the schedule in run_all):
  // if more than one workgroup's range holds part of it, add their pieces in
  // reduction order (workgroup order) and store the tile.  Workgroup w's tail
  // range is [w * Ut / G, (w + 1) * Ut / G); the owner of tail stage u is the last
  // w whose range starts at or before u.  With Ut >= G every range is non-empty,
  // the tile's pieces belong to owners w0..w1, and only w0's range can start
  // before the tile (its piece is then in its slot 1).  With Ut < G every range
  // holds at most one stage, so each of the tile's nst stages is its own piece,
  // in slot 0 of its owner.
  template <bool SH>
  __device__ __forceinline__ static void fixup(const FfnArgs& g, int* meta, int nb, int nbr, int G,
                                               int tq) {
    const int N = PHASE == 1 ? g.I : g.H;
    const int K = PHASE == 1 ? g.H : g.I;
    const int total = nb * ((N + BN - 1) / BN);
    const int nst = (K + BK - 1) / BK;
    const int F = total / G;
    const int r = total - F * G;
    if (tq >= r || !split_tail(r, G, F)) return;
    const int64_t Ut = (int64_t)r * nst;
    const int64_t ub = (int64_t)tq * nst;
    const int w0 = (int)(((ub + 1) * G - 1) / Ut);
    const int w1 = (int)(((ub + nst) * G - 1) / Ut);
    if (w0 == w1) return;  // one range holds the whole tile; run_all stored it
    const int t = F * G + tq;
    int rb, nt;
    tile_rc(t, nb, (N + BN - 1) / BN, rb, nt);
    const int64_t row0 = (int64_t)rb * BM;
    const int n0 = nt * BN;
    const int tid = threadIdx.x;
    // a launch of more than NT threads runs this too: the extra threads only
    // take part in the barrier
    const bool act = tid < NT;
    const int wave = act ? tid >> 6 : 0;
    const int lane = tid & 63;
    const int wk = wave % WK;
    const int wn = (wave / WK) % WN;
    const int wm = wave / (WK * WN);
    // The pieces in reduction order: (owner w, its piece slot).  The first one is
    // loaded before the tile's metadata, so the two memory round trips overlap.
    const bool w0_before = Ut >= G && (int64_t)w0 * Ut / G < ub;
    auto piece_of = [&](int q, int& w, int& pc) __attribute__((always_inline)) {
      if (Ut >= G) {
        w = w0 + q;
        pc = q == 0 && w0_before ? 1 : 0;
      } else {  // (u + 1) * G <= Ut * G < G * G fits 32 bits
        w = (int)(((unsigned)(ub + q + 1) * (unsigned)G - 1u) / (unsigned)Ut);
        pc = 0;
      }
    };
    const int npieces = Ut >= G ? w1 - w0 + 1 : nst;
    // A piece's fragments are loaded into their own registers, one piece ahead of
    // the additions: all of a piece's loads are in flight together, instead of one
    // wait per 16-byte load.  The pieces are still added in reduction order.
    f32x4 acc[NMAT][FM][FN], nxt[NMAT][FM][FN];
    auto fetch_piece = [&](int q) __attribute__((always_inline)) {
      int w, pc;
      piece_of(q, w, pc);
      const float* src = g.part + ((int64_t)w * 2 + pc) * PIECE + (wm * WN + wn) * NFRAG * 256;
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int jn = 0; jn < FN; ++jn)
            nxt[mt][i][jn] = *(const f32x4*)(src + (((mt * FM + i) * FN + jn) * 64 + lane) * 4);
    };
    if (act && wk == 0) fetch_piece(0);
    if (SH && rb >= nbr) {  // a shared expert's row-block (see run_all)
      const int Btok = g.slots / g.k;
      const int nbs = (Btok + BM - 1) / BM;
      if ((rb - nbr) / nbs >= g.n_shared) return;
      if (tid < BM) {
        const int t = ((rb - nbr) % nbs) * BM + tid;
        meta[tid] = t < Btok ? g.slots + t : -1;
      }
    } else {
      if ((unsigned)g.block_expert[rb] >= (unsigned)g.E_loc) return;
      if (tid < BM) {
        const int sl = g.sorted_slots[row0 + tid];
        meta[tid] = (sl >= 0 && sl < g.slots) ? sl : -1;
      }
    }
    __syncthreads();
    if (!act || wk != 0) return;
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jn = 0; jn < FN; ++jn) acc[mt][i][jn] = nxt[mt][i][jn];
    if (npieces > 1) fetch_piece(1);
    for (int q = 1; q < npieces; ++q) {
      f32x4 cur[NMAT][FM][FN];
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int jn = 0; jn < FN; ++jn) cur[mt][i][jn] = nxt[mt][i][jn];
      if (q + 1 < npieces) fetch_piece(q + 1);
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int jn = 0; jn < FN; ++jn) acc[mt][i][jn] = acc[mt][i][jn] + cur[mt][i][jn];
    }
    store_acc(g, acc, meta, row0, n0, wm, wn, lane);
  }
};

// ---------------------------------------------------------------------------
// configuration table: must match kVariants in moe_common.h
//   Cfg<V, PHASE, WKIND>::R is the tile runner of configuration V in that phase.
//   WIDE: the one-workgroup-per-CU class (else two per CU, 256 threads each); RX
//   multiplies the LDS row bytes of the fp32, fp8 and fp8 x fp8 tiles (their
//   fragments, decode or load shapes need 128-byte rows where the bf16 tile of the
//   wide class uses 64).
// ---------------------------------------------------------------------------
template <int V, int PHASE, int WKIND>
struct Cfg;
#define MOE_CFG(V, BM, BN1, BN2, ROWB1, ROWB2, WM, WN, WK, RS, STREAM, WIDE, RX)               \
  template <int PHASE, int WKIND>                                                             \
  struct Cfg<V, PHASE, WKIND> {                                                               \
    static constexpr int BN = PHASE == 1 ? BN1 : BN2;                                         \
    static constexpr int ROWB = (PHASE == 1 ? ROWB1 : ROWB2) * (WKIND == W_BF16 ? 1 : RX);    \
    static constexpr int WNX = (WIDE) && WKIND != W_BF16 ? 2 * (WN) : (WN);                   \
    using R = Tile<BM, BN, WM, WNX, WK, ROWB, RS, STREAM, PHASE, WKIND, 64 * (WM) * WNX * (WK), \
                   (WIDE) != 0>;                                                              \
  };                                                                                          \
  static_assert(kVariants[V].bm == BM && kVariants[V].bn1 == BN1 && kVariants[V].bn2 == BN2 && \
                    kVariants[V].rowb == ROWB1 && kVariants[V].wm == WM &&                    \
                    kVariants[V].wn == WN && kVariants[V].wk == WK && kVariants[V].splitk == 1 && \
                    kVariants[V].stream == STREAM &&                                          \
                    kVariants[V].wgcu == ((WIDE) ? 1 : kWgPerCu) &&                           \
                    ((WIDE) || 64 * (WM) * (WN) * (WK) == kThreads),                          \
                "kernel configuration table out of sync with kVariants");
// Streaming class: two workgroups share a compute unit, so each stage buffer
// holds at most 32 KiB: every stage carries 16 KiB of weights (the down phase has
// one weight matrix, so its LDS rows are twice as wide).  The small-M
// configurations read each weight tile once (one row-block per expert is the
// common case), so they stream the weights with non-temporal loads, which sustain
// a markedly higher HBM rate; the largest one serves many row-blocks per expert
// that re-read each weight tile from L2, so it keeps cached loads.
MOE_CFG(0, 16, 16, 16, 512, 1024, 1, 1, 4, 2, 1, 0, 1)
MOE_CFG(1, 32, 32, 32, 256, 512, 1, 2, 2, 2, 1, 0, 1)
MOE_CFG(2, 64, 64, 64, 128, 256, 2, 2, 1, 2, 1, 0, 1)
MOE_CFG(3, 128, 64, 128, 128, 128, 2, 2, 1, 2, 0, 0, 1)
// Wide class: one workgroup per compute unit computes a 256 x 256 output tile
// (gate/up: 128 gate and 128 up columns).  Per byte staged it does twice the MFMA
// work of the 128-row streaming tile, which halves the L2 and fabric traffic per
// FLOP where the matrix units bound the layer.  bf16 tiles: four waves, one per
// SIMD, of 128 x 128 each (their 256 fp32 sums per lane live in the accumulation
// registers), 32-deep stages (64-byte LDS rows, 32 KiB a stage).  fp32 and fp8
// tiles: eight waves of 128 x 64 (their register-staged path needs the second
// wave per SIMD to hide its loads), with 128-byte rows.
MOE_CFG(4, 256, 128, 256, 64, 64, 2, 2, 1, 2, 0, 1, 2)
// more of the streaming class: other column widths, stage depths and load policies
MOE_CFG(5, 16, 32, 32, 256, 512, 1, 2, 2, 2, 1, 0, 1)
MOE_CFG(6, 32, 16, 32, 512, 512, 1, 1, 4, 2, 1, 0, 1)
MOE_CFG(7, 64, 32, 64, 256, 256, 2, 2, 1, 2, 1, 0, 1)
MOE_CFG(8, 32, 64, 64, 128, 256, 1, 4, 1, 2, 1, 0, 1)
MOE_CFG(9, 64, 64, 64, 128, 256, 2, 2, 1, 2, 0, 0, 1)
MOE_CFG(10, 128, 64, 128, 128, 128, 2, 2, 1, 2, 1, 0, 1)
MOE_CFG(11, 32, 32, 32, 256, 512, 1, 2, 2, 2, 0, 0, 1)
#undef MOE_CFG
// the streaming class's entries, for the dispatch switches
#define MOE_STREAM_VARIANTS(X) X(0) X(1) X(2) X(3) X(5) X(6) X(7) X(8) X(9) X(10) X(11)

template <int PHASE, int WKIND>
constexpr int lds_bytes_stream() {
  int m = 0;
#define MOE_LDS(V)                                                                            \
  m = Cfg<V, PHASE, WKIND>::R::LDS_BYTES > m ? Cfg<V, PHASE, WKIND>::R::LDS_BYTES : m;
  MOE_STREAM_VARIANTS(MOE_LDS)
#undef MOE_LDS
  return m;
}
// threads per workgroup of the wide launch (and of the bf16 wide fix-up launch)
template <int WKIND>
constexpr int wide_threads() {
  return Cfg<kWideVariant, 1, WKIND>::R::THREADS;
}
static_assert(wide_threads<W_BF16>() == 64 * kVariants[kWideVariant].wm * kVariants[kWideVariant].wn,
              "the wide configuration's table entry describes its bf16 tiles");
// dynamic LDS of the wide launch; its bf16 tiles use four static stage buffers
template <int PHASE, int WKIND>
constexpr int lds_bytes_wide() {
  return WKIND == W_BF16 ? 0 : Cfg<kWideVariant, PHASE, WKIND>::R::LDS_BYTES;
}

// The tiles of configuration V in phase PHASE, dealt out statically over the
// launch's grid.
template <int V, int PHASE, int WKIND, bool SH>
__device__ __forceinline__ void run_phase(const FfnArgs& g, uint8_t* lds, int* meta3, int nb,
                                          int nbr) {
  using R = typename Cfg<V, PHASE, WKIND>::R;
  R::template run_all<SH>(g, lds, lds + R::STAGE, meta3, nb, nbr, xcd_slot(blockIdx.x, gridDim.x),
                          gridDim.x);
}

// Row-blocks of the launch: the routed ones the sort wrote (nbr), then with
// shared experts ceil(B / BM) per shared expert; none beyond the buffers.
template <bool SH>
__device__ __forceinline__ bool block_counts(const FfnArgs& g, int v, int& nb, int& nbr) {
  nbr = *g.num_blocks;
  if (v < 0 || v >= kNumVariants || nbr < 0 || (!SH && nbr == 0)) return false;
  const int bm = kVariants[v].bm;
  nb = nbr;
  if (SH) nb += g.n_shared * ((g.slots / g.k + bm - 1) / bm);
  // never address rows beyond the buffers, whatever the device state says
  const int nb_cap = (int)(g.rows_max / bm);
  nb = nb < nb_cap ? nb : nb_cap;
  nbr = nbr < nb ? nbr : nb;
  return nb > 0;
}

// The device status word: MOE_DEV_BAD_VARIANT for a configuration index outside
// the menu, MOE_DEV_BAD_BLOCKS for a row-block count below zero or beyond what the
// buffers hold (the launch then runs only the row-blocks that fit).  Workgroup 0
// of the streaming-class launch writes it once per phase, so each call reports
// its own inputs.
template <bool SH>
__device__ __forceinline__ void report_status(const FfnArgs& g, int v, int nbr) {
  if (blockIdx.x != 0 || threadIdx.x != 0 || g.status == nullptr) return;
  int st = 0;
  if (v < 0 || v >= kNumVariants) {
    st = MOE_DEV_BAD_VARIANT;
  } else {
    const int bm = kVariants[v].bm;
    int64_t nb = nbr;
    if (SH) nb += (int64_t)g.n_shared * ((g.slots / g.k + bm - 1) / bm);
    if (nbr < 0 || nb > g.rows_max / bm) st = MOE_DEV_BAD_BLOCKS;
  }
  *g.status = st;
}

// Streaming class: configurations 0-3, two 256-thread workgroups per CU.
template <int PHASE, int WKIND, bool SH>
__global__ void __launch_bounds__(kThreads, kWgPerCu) ffn_kernel(FfnArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int meta3[kMetaSlots * (kMaxBlockM + 4)];
  const int v = *g.variant;
  report_status<SH>(g, v, *g.num_blocks);
  int nb, nbr;
  if (v == kWideVariant || !block_counts<SH>(g, v, nb, nbr)) return;
  switch (v) {
#define MOE_RUN(V)                                         \
  case V:                                                  \
    run_phase<V, PHASE, WKIND, SH>(g, lds, meta3, nb, nbr); \
    break;
    MOE_STREAM_VARIANTS(MOE_RUN)
#undef MOE_RUN
    default: break;
  }
}

// The launch that follows the streaming one in each phase: one workgroup per CU
// (256 threads for bf16, 512 for fp32 and fp8).  With the wide configuration
// chosen it computes all of the phase's tiles; otherwise it is the streaming
// class's fix-up, adding the partial sums of each split tail tile (Tile::fixup;
// tail tile tq for tq = workgroup, workgroup + grid, ...).
template <int PHASE, int WKIND, bool SH>
__global__ void __launch_bounds__(wide_threads<WKIND>(), 1) ffn_wide_kernel(FfnArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int meta3[kMetaSlots * (kMaxBlockM + 4)];
  const int v = *g.variant;
  int nb, nbr;
  if (!block_counts<SH>(g, v, nb, nbr)) return;
  if (v == kWideVariant) {
    if constexpr (WKIND == W_BF16) {
      // four distinct LDS arrays: the compiler then waits for each stage's own
      // direct loads only (see Tile::run_dma)
      using R = typename Cfg<kWideVariant, PHASE, W_BF16>::R;
      __shared__ __attribute__((aligned(16))) uint8_t s0[R::STAGE];
      __shared__ __attribute__((aligned(16))) uint8_t s1[R::STAGE];
      __shared__ __attribute__((aligned(16))) uint8_t s2[R::STAGE];
      __shared__ __attribute__((aligned(16))) uint8_t s3[R::STAGE];
      __shared__ int pexp[kRunTable];
      __shared__ __attribute__((aligned(16))) uint8_t ostage[4 * R::OSTAGE];
      const int K = PHASE == 1 ? g.H : g.I;
      const int slot = xcd_slot(blockIdx.x, gridDim.x);
      // H and I are multiples of 128 (the API checks), so every reduction is whole
      // groups of four 32-deep stages
      if (K % (4 * R::BK) == 0 && K >= 4 * R::BK)
        R::template run_dma<SH, 4>(g, s0, s1, s2, s3, meta3, pexp, ostage, nb, nbr, slot, gridDim.x);
    } else {
      run_phase<kWideVariant, PHASE, WKIND, SH>(g, lds, meta3, nb, nbr);
    }
    return;
  }
  const int G = g.grid_stream;
  for (int tq = blockIdx.x; tq < G; tq += gridDim.x) {
    __syncthreads();  // the previous tail tile's readers of meta3 are done
    switch (v) {
#define MOE_FIX(V)                                                              \
  case V:                                                                       \
    Cfg<V, PHASE, WKIND>::R::template fixup<SH>(g, meta3, nb, nbr, G, tq); \
    break;
      MOE_STREAM_VARIANTS(MOE_FIX)
#undef MOE_FIX
      default: break;
    }
  }
}

// The fix-up launch of the wide class's split down-phase tail (Tile::wide_fixup):
// two workgroups per possible split tile (at most half the wide grid), one per
// half of the tile's rows.  It follows the wide launch on the stream, so the
// pieces are complete.
template <int PHASE, bool SH>
__global__ void __launch_bounds__(wide_threads<W_BF16>(), 1) ffn_wide_fixup_kernel(FfnArgs g, int grid_wide) {
  __shared__ int meta[kMaxBlockM + 4];
  __shared__ int pexp[kRunTable];
  const int v = *g.variant;
  if (v != kWideVariant) return;
  int nb, nbr;
  if (!block_counts<SH>(g, v, nb, nbr)) return;
  using R = typename Cfg<kWideVariant, PHASE, W_BF16>::R;
  const int K = PHASE == 1 ? g.H : g.I;
  if (K % (4 * R::BK) != 0 || K / R::BK < 8) return;  // no split below two four-stage groups
  R::template wide_fixup<SH>(g, meta, pexp, nb, nbr, grid_wide, blockIdx.x >> 1, blockIdx.x & 1);
}

// Whether the wide class can split the down phase's tail for this problem: the
// row-block count of its BLOCK_M is at most ceil(slots / BM) + min(E_loc, slots)
// (one partial block per active expert) plus the shared experts' blocks, and a
// split needs more tiles than one round.  Small problems skip the launch.
inline bool wide_split_possible(const FfnArgs& g, int grid_wide) {
  using R = Cfg<kWideVariant, 2, W_BF16>::R;
  const int64_t bm = kVariants[kWideVariant].bm;
  if (g.I % (4 * R::BK) != 0 || g.I / R::BK < 8) return false;
  const int64_t slots = g.slots;
  int64_t nb = (slots + bm - 1) / bm + (g.E_loc < slots ? g.E_loc : slots);
  if (nb > g.rows_max / bm) nb = g.rows_max / bm;
  if (g.n_shared > 0) nb += (int64_t)g.n_shared * ((slots / g.k + bm - 1) / bm);
  const int64_t bn = kVariants[kWideVariant].bn2;
  const int64_t ncol = (g.H + bn - 1) / bn;
  return nb * ncol > grid_wide && (int64_t)grid_wide * R::PIECE <= kPartBytes / 4;
}

template <int PHASE, int WKIND, bool SH>
hipError_t launch_phase_sh(const FfnArgs& g, int grid_wide, hipStream_t s) {
  constexpr int meta_bytes = kMetaSlots * (kMaxBlockM + 4) * 4;
  constexpr int lds = lds_bytes_stream<PHASE, WKIND>();
  static_assert((lds + meta_bytes) * kWgPerCu <= 160 * 1024, "LDS budget of kWgPerCu workgroups per CU");
  constexpr int ldsw = lds_bytes_wide<PHASE, WKIND>();
  constexpr int ldsw_static =
      WKIND == W_BF16 ? 4 * (Cfg<kWideVariant, PHASE, W_BF16>::R::STAGE + Cfg<kWideVariant, PHASE, W_BF16>::R::OSTAGE)
                      : 0;
  static_assert(ldsw + ldsw_static + meta_bytes + kRunTable * 4 <= 160 * 1024,
                "LDS budget of one wide workgroup per CU");
  hipError_t e = opt_in_lds((const void*)ffn_kernel<PHASE, WKIND, SH>, lds);
  if (e != hipSuccess) return e;
  e = opt_in_lds((const void*)ffn_wide_kernel<PHASE, WKIND, SH>, ldsw);
  if (e != hipSuccess) return e;
  ffn_kernel<PHASE, WKIND, SH><<<g.grid_stream, kThreads, lds, s>>>(g);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  ffn_wide_kernel<PHASE, WKIND, SH><<<grid_wide, wide_threads<WKIND>(), ldsw, s>>>(g);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (PHASE == 2 && WKIND == W_BF16) {
    if (wide_split_possible(g, grid_wide)) {
      ffn_wide_fixup_kernel<PHASE, SH><<<2 * ((grid_wide + 1) / 2), wide_threads<W_BF16>(), 0, s>>>(
          g, grid_wide);
      e = hipGetLastError();
    }
  }
  return e;
}

// the launch with shared experts is a separate instance, so that the routed-only
// kernels carry none of its code
template <int PHASE, int WKIND>
hipError_t launch_phase(const FfnArgs& g, int grid, hipStream_t s) {
  return g.n_shared > 0 ? launch_phase_sh<PHASE, WKIND, true>(g, grid, s)
                        : launch_phase_sh<PHASE, WKIND, false>(g, grid, s);
}

template <int WKIND>
hipError_t launch_w(const FfnArgs& g, int phases, int grid, hipStream_t s) {
  if (phases & 1) {
    const hipError_t e = launch_phase<1, WKIND>(g, grid, s);
    if (e != hipSuccess) return e;
  }
  if (phases & 2) return launch_phase<2, WKIND>(g, grid, s);
  return hipSuccess;
}

// Writes the wide configuration's packed weight copy (include/moe.h,
// moe_pack_wide): chunk q (16 bytes) of a region is bytes 16 (q % 4) .. of row
// (q / 4) % 256 of block q / 1024; a block is one 32-deep stage of one expert's
// column tile (gate/up: rows 0-127 from W1, 128-255 from W3; down: W2), and rows
// past the matrix's end are zeros.
__global__ void __launch_bounds__(256) pack_wide_kernel(const uint16_t* w1, const uint16_t* w3,
                                                        const uint16_t* w2, u32x4* out, int E, int H,
                                                        int I) {
  const int64_t ncol1 = (I + 127) / 128, nst1 = H / 32, ncol2 = (H + 255) / 256, nst2 = I / 32;
  const int64_t n1 = (int64_t)E * ncol1 * nst1 * 1024;
  const int64_t n2 = (int64_t)E * ncol2 * nst2 * 1024;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n1 + n2;
       q += (int64_t)gridDim.x * blockDim.x) {
    const bool gu = q < n1;
    const int64_t qq = gu ? q : q - n1;
    const int64_t blk = qq >> 10;
    const int r = (int)((qq >> 2) & 255), c = (int)(qq & 3);
    const int64_t nst = gu ? nst1 : nst2, ncol = gu ? ncol1 : ncol2;
    const int64_t kb = blk % nst, nt = (blk / nst) % ncol, e = blk / (nst * ncol);
    const uint16_t* src = gu ? (r < 128 ? w1 : w3) : w2;
    const int64_t row = gu ? nt * 128 + (r & 127) : nt * 256 + r;
    const int64_t N = gu ? I : H, K = gu ? H : I;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < N) v = *(const u32x4*)(src + (e * N + row) * K + kb * 32 + c * 8);
    out[q] = v;
  }
}

}  // namespace

int64_t pack_wide_bytes(const moe_problem& p) {
  const int64_t E = (int64_t)p.local_experts + p.shared_experts;
  const int64_t H = p.hidden, I = p.inter;
  return 2 * E * ((I + 127) / 128 * 128) * H * 2 + E * ((H + 255) / 256 * 256) * I * 2;
}

hipError_t launch_pack_wide(const moe_problem& p, const void* w1, const void* w3, const void* w2,
                            void* packed, hipStream_t s) {
  const int64_t chunks = pack_wide_bytes(p) / 16;
  const int64_t want = (chunks + 255) / 256;
  const int grid = (int)(want < 4096 ? want : 4096);
  pack_wide_kernel<<<grid, 256, 0, s>>>((const uint16_t*)w1, (const uint16_t*)w3, (const uint16_t*)w2,
                                        (u32x4*)packed, p.local_experts + p.shared_experts, p.hidden,
                                        p.inter);
  return hipGetLastError();
}

hipError_t launch_grouped_ffn(const moe_problem& p, int phases, const void* x, const uint8_t* xq,
                              const float* xs, const uint8_t* hq, const float* hs, const void* w1,
                              const void* w3, const void* w2, const float* s1, const float* s3,
                              const float* s2, const int32_t* sorted_slots,
                              const int32_t* block_expert, const int32_t* num_blocks,
                              const int32_t* variant, void* y_slots, void* h, float* part,
                              int32_t* status, int num_cus, int64_t rows_max, hipStream_t s) {
  const int grid_stream = num_cus * kWgPerCu < kMaxGrid ? num_cus * kWgPerCu : kMaxGrid;
  const int grid = num_cus < kMaxGrid ? num_cus : kMaxGrid;  // the wide class's launch
  FfnArgs g{x, w1, w3, w2, s1, s3, s2, sorted_slots, block_expert, num_blocks, variant,
            h, y_slots, part, p.hidden, p.inter, p.top_k, p.local_experts,
            p.tokens * p.top_k, rows_max, nullptr, p.shared_experts, status, grid_stream,
            (const uint8_t*)p.packed_weights};
  switch (p.weight_dtype) {
    case MOE_F32: return launch_w<W_F32>(g, phases, grid, s);
    case MOE_BF16: return launch_w<W_BF16>(g, phases, grid, s);
    case MOE_FP8_E4M3:
      if (p.act_quant) {  // gate/up on fp8 x fp8; the down phase as for fp8 weights
        if (phases & 1) {
          FfnArgs gq = g;
          gq.x = xq;
          gq.xs = xs;
          const hipError_t e = launch_phase<1, W_FP8A>(gq, grid, s);
          if (e != hipSuccess) return e;
        }
        if (!(phases & 2)) return hipSuccess;
        if (p.act_quant == 2) {  // down on fp8 h x fp8 weights; output y_slots
          FfnArgs gh = g;
          gh.h = const_cast<uint8_t*>(hq);  // read only in the down phase
          gh.xs = hs;
          return launch_phase<2, W_FP8A>(gh, grid, s);
        }
        return launch_phase<2, W_FP8>(g, grid, s);
      }
      return launch_w<W_FP8>(g, phases, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
