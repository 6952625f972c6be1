// moe_common.h -- shared device/host definitions of the gfx950 fused-MoE library.
// Internal header of the GPU library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// vector types
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kWave = 64;

// bf16 <-> f32 (round to nearest even; inputs are finite in this library)
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(r >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------------------
// Compiled tile configurations of the polymorphic grouped FFN.  They come in two
// occupancy classes, each one kernel per GEMM phase with one workgroup size, one
// LDS allocation and one register budget for all its entries (RaMP, section 3.3:
// one shared-memory buffer and one register count for every entry of a
// polymorphic kernel):
//   - the streaming class: 256 threads, two workgroups per CU;
//   - the wide class: one workgroup per CU, a 256 x 256 output tile whose larger
//     per-workgroup reuse of every staged byte suits the loads where the matrix
//     units, not HBM, bound the time (entry 4).  Its bf16 tiles run four waves
//     (the wave counts below); its fp32 and fp8 tiles run eight, twice the waves
//     along N.
//   bm    token rows per tile (b_c of RaMP Eq. 1)
//   bn1   weight rows per tile of W1 and of W3 in the gate/up phase
//   bn2   weight rows per tile of W2 in the down phase
//   rowb  LDS bytes per tile row per pipeline stage for bf16 operands (BLOCK_K =
//         rowb / 2; fp32 operands use half the depth, and in the wide class the
//         fp32 and fp8 x fp8 tiles use twice the row bytes)
//   wm, wn, wk  waves along M, along N, and splitting K inside a tile (bf16)
//   splitk      tiles splitting K of the down phase (1 = none)
//   stream      1: weights are read with non-temporal (streaming) loads, for the
//               small-M configurations where each weight tile is read once;
//               0: cached loads, for row-blocks that re-read a weight tile
//   wgcu        workgroups per CU (2: streaming class, 1: wide class)
// ---------------------------------------------------------------------------
struct VariantDesc {
  int bm, bn1, bn2, rowb, wm, wn, wk, splitk, stream, wgcu;
};

constexpr int kNumVariants = 12;
constexpr int kThreads = 256;  // streaming class
constexpr int kWideVariant = 4;

// The compiled configuration space.  The served menu of a workload is chosen
// from it offline (RaMP section 3.1: greedily, on timed fit loads); entries left
// out of a menu get a cost-model prediction that never wins.
constexpr VariantDesc kVariants[kNumVariants] = {
    {16, 16, 16, 512, 1, 1, 4, 1, 1, 2},      // 0
    {32, 32, 32, 256, 1, 2, 2, 1, 1, 2},      // 1
    {64, 64, 64, 128, 2, 2, 1, 1, 1, 2},      // 2
    {128, 64, 128, 128, 2, 2, 1, 1, 0, 2},    // 3
    {256, 128, 256, 64, 2, 2, 1, 1, 0, 1},    // 4: the wide class (bf16 waves)
    {16, 32, 32, 256, 1, 2, 2, 1, 1, 2},      // 5: 0 with twice the columns
    {32, 16, 32, 512, 1, 1, 4, 1, 1, 2},      // 6: 1 with half the gate/up columns
    {64, 32, 64, 256, 2, 2, 1, 1, 1, 2},      // 7: 2 with half the gate/up columns
    {32, 64, 64, 128, 1, 4, 1, 1, 1, 2},      // 8: 1 with twice the columns
    {64, 64, 64, 128, 2, 2, 1, 1, 0, 2},      // 9: 2 with cached weight loads
    {128, 64, 128, 128, 2, 2, 1, 1, 1, 2},    // 10: 3 with streaming weight loads
    {32, 32, 32, 256, 1, 2, 2, 1, 0, 2},      // 11: 1 with cached weight loads
};

constexpr int kMinBlockM = 16;
constexpr int kMaxBlockM = 256;

// workgroups per CU of the streaming class's persistent launch
constexpr int kWgPerCu = 2;

// The streaming class's persistent grid is min(CUs * kWgPerCu, kMaxGrid)
// workgroups (MI355X: 256 CUs, so 512); the wide class's is min(CUs, kMaxGrid).
// In the streaming class each workgroup may leave up to two partial tiles of at
// most kPieceMax fp32 sums in the workspace (the split tail tiles; the wide class
// never splits a tile), so the workspace size does not depend on the device.
constexpr int kMaxGrid = 512;
constexpr int piece_floats(const VariantDesc& d) {
  return 2 * d.bm * d.bn1 > d.bm * d.bn2 ? 2 * d.bm * d.bn1 : d.bm * d.bn2;
}
constexpr int piece_max() {
  int m = 0;
  for (int v = 0; v < kNumVariants; ++v)
    if (kVariants[v].wgcu == kWgPerCu) m = piece_floats(kVariants[v]) > m ? piece_floats(kVariants[v]) : m;
  return m;
}
constexpr int kPieceMax = piece_max();
constexpr int64_t kPartBytes = (int64_t)kMaxGrid * 2 * kPieceMax * 4;

// Device-side table of the cost-model constants (RaMP Eq. 1) per configuration.
// With shared experts, each adds ceil(B / b) row-tiles (rt_shared) and one active
// expert (a_shared) to the features of every configuration.
struct CostTable {
  int32_t b[kNumVariants];
  int32_t q1[kNumVariants];
  int32_t q2[kNumVariants];
  int32_t S1[kNumVariants];
  int32_t S2[kNumVariants];
  int32_t rt_shared[kNumVariants];
  int32_t a_shared;
};

constexpr int kMaxShared = 8;

// Raises the dynamic-LDS limit of kernel `fn` on the current device to at least
// `bytes`: one hipFuncSetAttribute per kernel and device, safe to call from
// several host threads at once.
hipError_t opt_in_lds(const void* fn, int bytes);
// Compute units of the current device, queried once per device (thread-safe).
hipError_t device_cus(int* cus);

// Host-side launchers (one per translation unit).
hipError_t launch_route_topk(const moe_problem& p, const float* logits, int32_t* ids, float* w,
                             int32_t* counts, hipStream_t s);
hipError_t launch_select_config(const moe_problem& p, const int32_t* counts, const float* theta,
                                const CostTable& tab, int32_t* variant, float* t_hat,
                                hipStream_t s);
hipError_t launch_align_sort(const moe_problem& p, const int32_t* ids, const int32_t* variant,
                             int32_t* sorted_slots, int32_t* block_expert, int32_t* num_blocks,
                             int32_t* slot_pos, hipStream_t s);
hipError_t launch_route_select_align(const moe_problem& p, const float* logits,
                                     const float* theta, const CostTable& tab, int32_t* ids,
                                     float* w, int32_t* counts, int32_t* variant, float* t_hat,
                                     int32_t* sorted_slots, int32_t* block_expert,
                                     int32_t* num_blocks, int32_t* slot_pos, hipStream_t s);
// FP8 activation quantization: xq [B][H] E4M3FN codes, xs [B][H/128] scales
hipError_t launch_quant_act(const moe_problem& p, const void* x, uint8_t* xq, float* xs,
                            hipStream_t s);
// the same for the rows of h [rows_max][I] that hold a slot, among the rows the
// chosen configuration's row-blocks cover (read from device memory)
hipError_t launch_quant_h(const moe_problem& p, const void* h, uint8_t* hq, float* hs,
                          const int32_t* sorted_slots, const int32_t* num_blocks,
                          const int32_t* variant, int64_t rows_max, hipStream_t s);
// phases: 1 = gate/up + SwiGLU only, 2 = down only, 3 = both (two launches).
// With p.act_quant the gate/up phase reads the quantized x (xq, xs) instead of x,
// and with act_quant 2 the down phase reads the quantized h (hq, hs).
// status: the device status word (MOE_DEV_* bits), written by workgroup 0 of
// every grouped-FFN launch.
hipError_t launch_grouped_ffn(const moe_problem& p, int phases, const void* x, const uint8_t* xq,
                              const float* xs, const uint8_t* hq, const float* hs, const void* w1,
                              const void* w3, const void* w2, const float* s1, const float* s3,
                              const float* s2, const int32_t* sorted_slots,
                              const int32_t* block_expert, const int32_t* num_blocks,
                              const int32_t* variant, void* y_slots, void* h, float* part,
                              int32_t* status, int num_cus, int64_t rows_max, hipStream_t s);
// The wide configuration's packed weight copy (include/moe.h, moe_pack_wide):
// its size in bytes, and the launch that writes it from W1, W3, W2.
int64_t pack_wide_bytes(const moe_problem& p);
hipError_t launch_pack_wide(const moe_problem& p, const void* w1, const void* w3, const void* w2,
                            void* packed, hipStream_t s);
// num_blocks / variant: device values of the sort, needed with shared experts only
hipError_t launch_combine(const moe_problem& p, const void* y_slots, const int32_t* slot_pos,
                          const float* w, const int32_t* num_blocks, const int32_t* variant,
                          void* y, int64_t rows_max, hipStream_t s);


}  // namespace moe
