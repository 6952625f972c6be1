// moe_api.hip -- the C ABI of the fused-MoE library: host-side validation, buffer
// sizing and kernel enqueue.  No call allocates, frees, synchronises or reads device
// memory from the host, so every call can be captured into a HIP graph.
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <utility>

#include "fused_ffn.h"
#include "moe_common.h"

namespace moe {
size_t align_lds_bytes(int B, int E_loc);

hipError_t opt_in_lds(const void* fn, int bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> granted;  // (kernel, device) -> bytes
  std::lock_guard<std::mutex> lock(mu);
  int& have = granted[{fn, dev}];
  if (have >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) have = bytes;
  return e;
}

hipError_t device_cus(int* cus) {
  static std::atomic<int> cache[64];  // zero-initialised: 0 = not yet queried
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return hipSuccess;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n <= 0) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return hipSuccess;
}
}  // namespace moe

using namespace moe;

namespace {

// workspace: a 256-byte header (the device status word at offset 0, then
// reserved bytes), h, then the partial tiles
constexpr int64_t kWsHeader = 256;
constexpr size_t kMaxLds = 160 * 1024;

int elem_bytes(int dt) { return dt == MOE_F32 ? 4 : (dt == MOE_BF16 ? 2 : 1); }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// rows of sorted_slots / h / y_slots: every routed slot, padding of at most
// BLOCK_M - 1 rows per active expert, and each shared expert's B rows plus padding
int64_t rows_max_of(const moe_problem* p) {
  const int64_t slots = (int64_t)p->tokens * p->top_k;
  const int64_t active_max = slots < p->local_experts ? slots : p->local_experts;
  return slots + active_max * (kMaxBlockM - 1) +
         (int64_t)p->shared_experts * ((int64_t)p->tokens + kMaxBlockM - 1);
}

moe_status validate(const moe_problem* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  if (p->tokens < 1 || p->hidden < 128 || p->inter < 128) return MOE_ERR_INVALID_ARG;
  if (p->hidden % 128 || p->inter % 128) return MOE_ERR_INVALID_ARG;
  if (p->num_experts < 1 || p->num_experts > 4096) return MOE_ERR_INVALID_ARG;
  if (p->expert_begin < 0 || p->local_experts < 1 || p->local_experts > 1024) return MOE_ERR_INVALID_ARG;
  if ((int64_t)p->expert_begin + p->local_experts > p->num_experts) return MOE_ERR_INVALID_ARG;
  if (p->top_k < 1 || p->top_k > 32 || p->top_k > p->num_experts) return MOE_ERR_INVALID_ARG;
  if (p->renormalize != 0 && p->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (p->act_quant < 0 || p->act_quant > 2) return MOE_ERR_INVALID_ARG;
  if (p->shared_experts < 0 || p->shared_experts > kMaxShared) return MOE_ERR_INVALID_ARG;
  const int a = p->act_dtype, w = p->weight_dtype;
  if (a < MOE_F32 || a > MOE_FP8_E4M3 || w < MOE_F32 || w > MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  const bool ok = (a == MOE_F32 && w == MOE_F32) || (a == MOE_BF16 && w == MOE_BF16) ||
                  (a == MOE_BF16 && w == MOE_FP8_E4M3);
  if (!ok) return MOE_ERR_UNSUPPORTED;
  // the FP8 activation path: bf16 activations quantized for fp8-weight GEMMs
  if (p->act_quant && !(a == MOE_BF16 && w == MOE_FP8_E4M3)) return MOE_ERR_UNSUPPORTED;
  // the wide configuration's packed weight copy: bf16 problems only
  if (p->packed_weights && (!(a == MOE_BF16 && w == MOE_BF16) || !aligned(p->packed_weights, 256)))
    return MOE_ERR_INVALID_ARG;
  // 32-bit slot and row indices
  const int64_t slots = (int64_t)p->tokens * p->top_k;
  if (slots >= (1ll << 30)) return MOE_ERR_UNSUPPORTED;
  // the alignment step keeps its tables in one workgroup's LDS
  if (align_lds_bytes(p->tokens, p->local_experts) > kMaxLds - 512) return MOE_ERR_UNSUPPORTED;
  // the grouped FFN addresses x, h, y_slots and one expert's weight matrix with
  // 32-bit byte offsets below 2^31 (buffer loads; offsets from 2^31 up mark
  // chunks with no operand)
  {
    const int64_t rmax = rows_max_of(p);
    const int64_t wide = p->hidden > p->inter ? p->hidden : p->inter;
    const int64_t ab = elem_bytes(a), wb = elem_bytes(w);
    if (rmax * wide * ab >= (1ll << 31) || (int64_t)p->tokens * p->hidden * ab >= (1ll << 31) ||
        (int64_t)p->inter * p->hidden * wb >= (1ll << 31))
      return MOE_ERR_UNSUPPORTED;
  }
  // the cost model converts tile and wave counts to fp32 exactly (< 2^24)
  const int64_t rows = rows_max_of(p);
  for (int v = 0; v < kNumVariants; ++v) {
    const int64_t rt = rows / kVariants[v].bm;
    const int64_t q1 = (p->inter + kVariants[v].bn1 - 1) / kVariants[v].bn1;
    const int64_t q2 = (p->hidden + kVariants[v].bn2 - 1) / kVariants[v].bn2 * kVariants[v].splitk;
    const int64_t T = rt * (q1 + q2);
    if (T >= (1ll << 24)) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// codes and scales of n rows of m columns, each rounded up to 256 bytes
int64_t codes_bytes(int64_t n, int64_t m) { return (n * m + 255) / 256 * 256; }
int64_t scales_bytes(int64_t n, int64_t m) { return (n * (m / 128) * 4 + 255) / 256 * 256; }


// x codes and scales (act_quant >= 1), then h codes and scales (act_quant == 2)
int64_t quant_bytes(const moe_problem* p) {
  int64_t b = 0;
  if (p->act_quant >= 1) b += codes_bytes(p->tokens, p->hidden) + scales_bytes(p->tokens, p->hidden);
  if (p->act_quant == 2) {
    const int64_t r = rows_max_of(p);
    b += codes_bytes(r, p->inter) + scales_bytes(r, p->inter);
  }
  return b;
}

void sizes_of(const moe_problem* p, moe_sizes* s) {
  const int64_t slots = (int64_t)p->tokens * p->top_k;
  const int64_t active_max = slots < p->local_experts ? slots : p->local_experts;
  s->rows_max = rows_max_of(p);
  s->blocks_max = s->rows_max / kMinBlockM + 1;
  const int eb = elem_bytes(p->act_dtype);
  s->y_slots_bytes = s->rows_max * p->hidden * eb;
  int64_t hb = s->rows_max * p->inter * eb;
  hb = (hb + 255) / 256 * 256;
  s->workspace_bytes = kWsHeader + hb + quant_bytes(p) + kPartBytes;
  s->align_ws_bytes = 0;
}

// workspace layout: header | h | (act_quant) xq [B][H] u8, xs [B][H/128] f32 | parts
int64_t h_bytes(const moe_problem* p, int64_t rows_max) {
  const int64_t hb = rows_max * p->inter * elem_bytes(p->act_dtype);
  return (hb + 255) / 256 * 256;
}


int num_cus_current(hipError_t* err) {
  int n = 0;
  *err = device_cus(&n);
  return *err == hipSuccess ? n : 0;
}

moe_status fill_cost_table(const moe_problem* p, CostTable* t) {
  hipError_t err;
  const int cus = num_cus_current(&err);
  if (err != hipSuccess || cus <= 0) return MOE_ERR_HIP;
  for (int v = 0; v < kNumVariants; ++v) {
    t->b[v] = kVariants[v].bm;
    // column tiles per row-block (a wide tile may reach past H: ragged last tile)
    t->q1[v] = (p->inter + kVariants[v].bn1 - 1) / kVariants[v].bn1;
    t->q2[v] = (p->hidden + kVariants[v].bn2 - 1) / kVariants[v].bn2 * kVariants[v].splitk;
    // tiles resident at once: the persistent grid of the configuration's class
    const int per_cu = kVariants[v].wgcu;
    const int grid = cus * per_cu < kMaxGrid ? cus * per_cu : kMaxGrid;
    t->S1[v] = grid;
    t->S2[v] = grid;
    t->rt_shared[v] = p->shared_experts * ((p->tokens + kVariants[v].bm - 1) / kVariants[v].bm);
  }
  t->a_shared = p->shared_experts;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return 8; }

moe_status moe_query_sizes(const moe_problem* p, moe_sizes* out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  const moe_status st = validate(p);
  if (st != MOE_OK) return st;
  sizes_of(p, out);
  return MOE_OK;
}

int32_t moe_num_variants(void) { return kNumVariants; }

moe_status moe_variant_info(int32_t v, int32_t* out) {
  if (!out || v < 0 || v >= kNumVariants) return MOE_ERR_INVALID_ARG;
  const VariantDesc& d = kVariants[v];
  const int32_t vals[MOE_VARIANT_FIELDS] = {d.bm,     d.bn1,    d.bn2,  d.rowb / 2,
                                            d.wm,     d.wn,     d.wk,   d.splitk,
                                            d.stream, d.wgcu,   64 * d.wm * d.wn * d.wk};
  memcpy(out, vals, sizeof vals);
  return MOE_OK;
}

moe_status moe_cost_constants(const moe_problem* p, int32_t* b, int32_t* q1, int32_t* q2,
                              int32_t* S1, int32_t* S2) {
  if (!b || !q1 || !q2 || !S1 || !S2) return MOE_ERR_INVALID_ARG;
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  CostTable t;
  st = fill_cost_table(p, &t);
  if (st != MOE_OK) return st;
  for (int v = 0; v < kNumVariants; ++v) {
    b[v] = t.b[v];
    q1[v] = t.q1[v];
    q2[v] = t.q2[v];
    S1[v] = t.S1[v];
    S2[v] = t.S2[v];
  }
  return MOE_OK;
}

moe_status moe_route_topk(const moe_problem* p, const float* logits, int32_t* topk_ids,
                          float* topk_w, int32_t* counts, void* stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (!logits || !topk_ids || !topk_w || !counts) return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(counts, 4))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_route_topk(*p, logits, topk_ids, topk_w, counts, (hipStream_t)stream));
}

moe_status moe_select_config(const moe_problem* p, const int32_t* counts, const float* theta,
                             int32_t* variant, float* t_hat, void* stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (!counts || !theta || !variant) return MOE_ERR_INVALID_ARG;
  CostTable t;
  st = fill_cost_table(p, &t);
  if (st != MOE_OK) return st;
  return hip_status(launch_select_config(*p, counts, theta, t, variant, t_hat, (hipStream_t)stream));
}

moe_status moe_align_sort(const moe_problem* p, const int32_t* topk_ids, const int32_t* variant,
                          int32_t* sorted_slots, int32_t* block_expert, int32_t* num_blocks,
                          int32_t* slot_pos, void* stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (!topk_ids || !variant || !sorted_slots || !block_expert || !num_blocks || !slot_pos)
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_align_sort(*p, topk_ids, variant, sorted_slots, block_expert,
                                      num_blocks, slot_pos, (hipStream_t)stream));
}

moe_status moe_route_select_align(const moe_problem* p, const float* logits, const float* theta,
                                  int32_t* topk_ids, float* topk_w, int32_t* counts,
                                  int32_t* variant, float* t_hat, int32_t* sorted_slots,
                                  int32_t* block_expert, int32_t* num_blocks, int32_t* slot_pos,
                                  void* stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (!logits || !topk_ids || !topk_w || !counts || !variant || !sorted_slots || !block_expert ||
      !num_blocks || !slot_pos)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(counts, 4))
    return MOE_ERR_INVALID_ARG;
  CostTable t;
  st = fill_cost_table(p, &t);
  if (st != MOE_OK) return st;
  return hip_status(launch_route_select_align(*p, logits, theta, t, topk_ids, topk_w, counts,
                                              variant, t_hat, sorted_slots, block_expert,
                                              num_blocks, slot_pos, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Shared validation and enqueue of the grouped FFN entry points.  phases: 1 gate/up
// (needs x, w1, w3, s1, s3), 2 down (needs w2, s2, y_slots), 3 both.
moe_status grouped_ffn_phases(int phases, const moe_problem* p, const void* x, const void* w1,
                              const void* w3, const void* w2, const float* s1, const float* s3,
                              const float* s2, const int32_t* sorted_slots,
                              const int32_t* block_expert, const int32_t* num_blocks,
                              const int32_t* variant, void* y_slots, void* workspace,
                              size_t workspace_bytes, void* stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  const bool up = phases & 1, down = phases & 2;
  const bool fp8 = p->weight_dtype == MOE_FP8_E4M3;
  if (!sorted_slots || !block_expert || !num_blocks || !variant || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (up && (!x || !w1 || !w3 || (fp8 && (!s1 || !s3)))) return MOE_ERR_INVALID_ARG;
  if (down && (!w2 || !y_slots || (fp8 && !s2))) return MOE_ERR_INVALID_ARG;
  if (up && (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w3, 16) ||
             (fp8 && (!aligned(s1, 4) || !aligned(s3, 4)))))
    return MOE_ERR_INVALID_ARG;
  if (down && (!aligned(w2, 16) || !aligned(y_slots, 16) || (fp8 && !aligned(s2, 4))))
    return MOE_ERR_INVALID_ARG;
  if (!aligned(workspace, 256)) return MOE_ERR_INVALID_ARG;
  moe_sizes sz;
  sizes_of(p, &sz);
  if ((int64_t)workspace_bytes < sz.workspace_bytes) return MOE_ERR_WORKSPACE;
  hipError_t err;
  const int cus = num_cus_current(&err);
  if (err != hipSuccess || cus <= 0) return MOE_ERR_HIP;
  int32_t* status = (int32_t*)((char*)workspace + MOE_DEVICE_STATUS_OFFSET);
  void* h = (char*)workspace + kWsHeader;
  float* part = (float*)((char*)workspace + (sz.workspace_bytes - kPartBytes));
  uint8_t* xq = nullptr;
  float* xs = nullptr;
  uint8_t* hq = nullptr;
  float* hs = nullptr;
  if (p->act_quant) {
    xq = (uint8_t*)workspace + kWsHeader + h_bytes(p, sz.rows_max);
    xs = (float*)(xq + codes_bytes(p->tokens, p->hidden));
    if (p->act_quant == 2) {
      hq = (uint8_t*)xs + scales_bytes(p->tokens, p->hidden);
      hs = (float*)(hq + codes_bytes(sz.rows_max, p->inter));
    }
    if (up) {
      const hipError_t e = launch_quant_act(*p, x, xq, xs, (hipStream_t)stream);
      if (e != hipSuccess) return MOE_ERR_HIP;
    }
  }
  if (up && down) {  // two calls, so that h is quantized between the phases
    const moe_status st1 = hip_status(launch_grouped_ffn(
        *p, 1, x, xq, xs, nullptr, nullptr, w1, w3, w2, fp8 ? s1 : nullptr, fp8 ? s3 : nullptr,
        fp8 ? s2 : nullptr, sorted_slots, block_expert, num_blocks, variant, y_slots, h, part,
        status, cus, sz.rows_max, (hipStream_t)stream));
    if (st1 != MOE_OK) return st1;
  }
  if (down && p->act_quant == 2) {
    const hipError_t e = launch_quant_h(*p, h, hq, hs, sorted_slots, num_blocks, variant,
                                        sz.rows_max, (hipStream_t)stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (up && down) phases = 2;
  return hip_status(launch_grouped_ffn(*p, phases, x, xq, xs, hq, hs, w1, w3, w2, fp8 ? s1 : nullptr,
                                       fp8 ? s3 : nullptr, fp8 ? s2 : nullptr, sorted_slots,
                                       block_expert, num_blocks, variant, y_slots, h, part, status,
                                       cus, sz.rows_max, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// The library-owned workspace of moe_grouped_ffn_noalloc: one array per GPU,
// reserved when the library's code object is loaded on that GPU and held until the
// process ends.  In host code `scratch` is only a stand-in for the array: its
// device address comes from hipGetSymbolAddress, once per device, with that device
// current, and only that address is ever passed to kernels.
// ---------------------------------------------------------------------------
constexpr int64_t kScratchBytes = 256ll << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];
std::mutex scratch_mu;

hipError_t scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = scratch_addr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    ptr = scratch_addr[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (ptr == nullptr || ((uintptr_t)ptr & 255) != 0) return hipErrorInvalidSymbol;
      scratch_addr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return hipSuccess;
}

}  // namespace

extern "C" {

moe_status moe_grouped_ffn_noalloc(const moe_problem* p, const void* x, const void* w1,
                                   const void* w3, const void* w2, const float* s1,
                                   const float* s3, const float* s2, const int32_t* sorted_slots,
                                   const int32_t* block_expert, const int32_t* num_blocks,
                                   const int32_t* variant, void* y_slots, void* stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  moe_sizes sz;
  sizes_of(p, &sz);
  if (sz.workspace_bytes > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_of_current_device(&ws) != hipSuccess) return MOE_ERR_HIP;
  return grouped_ffn_phases(3, p, x, w1, w3, w2, s1, s3, s2, sorted_slots, block_expert,
                            num_blocks, variant, y_slots, ws, (size_t)kScratchBytes, stream);
}

int64_t moe_noalloc_workspace_limit(void) { return kScratchBytes; }

moe_status moe_pack_wide_bytes(const moe_problem* p, int64_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  const moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (p->act_dtype != MOE_BF16 || p->weight_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  *bytes = pack_wide_bytes(*p);
  return MOE_OK;
}

moe_status moe_pack_wide(const moe_problem* p, const void* w1, const void* w3, const void* w2,
                         void* packed, void* stream) {
  const moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (p->act_dtype != MOE_BF16 || p->weight_dtype != MOE_BF16 || p->packed_weights) return MOE_ERR_INVALID_ARG;
  if (!w1 || !w3 || !w2 || !packed || !aligned(packed, 256) || !aligned(w1, 16) || !aligned(w3, 16) ||
      !aligned(w2, 16))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_pack_wide(*p, w1, w3, w2, packed, (hipStream_t)stream));
}

moe_status moe_grouped_ffn(const moe_problem* p, const void* x, const void* w1, const void* w3,
                           const void* w2, const float* s1, const float* s3, const float* s2,
                           const int32_t* sorted_slots, const int32_t* block_expert,
                           const int32_t* num_blocks, const int32_t* variant, void* y_slots,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return grouped_ffn_phases(3, p, x, w1, w3, w2, s1, s3, s2, sorted_slots, block_expert,
                            num_blocks, variant, y_slots, workspace, workspace_bytes, stream);
}

moe_status moe_grouped_gate_up(const moe_problem* p, const void* x, const void* w1,
                               const void* w3, const float* s1, const float* s3,
                               const int32_t* sorted_slots, const int32_t* block_expert,
                               const int32_t* num_blocks, const int32_t* variant, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return grouped_ffn_phases(1, p, x, w1, w3, nullptr, s1, s3, nullptr, sorted_slots,
                            block_expert, num_blocks, variant, nullptr, workspace,
                            workspace_bytes, stream);
}

moe_status moe_grouped_down(const moe_problem* p, const void* w2, const float* s2,
                            const int32_t* sorted_slots, const int32_t* block_expert,
                            const int32_t* num_blocks, const int32_t* variant, void* y_slots,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return grouped_ffn_phases(2, p, nullptr, nullptr, nullptr, w2, nullptr, nullptr, s2,
                            sorted_slots, block_expert, num_blocks, variant, y_slots, workspace,
                            workspace_bytes, stream);
}

moe_status moe_quant_act(const moe_problem* p, const void* x, uint8_t* xq, float* xs,
                         void* stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (!p->act_quant) return MOE_ERR_INVALID_ARG;
  if (!x || !xq || !xs) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(xq, 8) || !aligned(xs, 4)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quant_act(*p, x, xq, xs, (hipStream_t)stream));
}

moe_status moe_combine(const moe_problem* p, const void* y_slots, const int32_t* slot_pos,
                       const float* topk_w, void* y, void* stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (p->shared_experts) return MOE_ERR_INVALID_ARG;
  if (!y_slots || !slot_pos || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned(y_slots, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
  moe_sizes sz;
  sizes_of(p, &sz);
  return hip_status(launch_combine(*p, y_slots, slot_pos, topk_w, nullptr, nullptr, y, sz.rows_max,
                                   (hipStream_t)stream));
}

moe_status moe_combine_shared(const moe_problem* p, const void* y_slots, const int32_t* slot_pos,
                              const float* topk_w, const int32_t* num_blocks,
                              const int32_t* variant, void* y, void* stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  if (!p->shared_experts) return MOE_ERR_INVALID_ARG;
  if (!y_slots || !slot_pos || !topk_w || !y || !num_blocks || !variant) return MOE_ERR_INVALID_ARG;
  if (!aligned(y_slots, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
  moe_sizes sz;
  sizes_of(p, &sz);
  return hip_status(launch_combine(*p, y_slots, slot_pos, topk_w, num_blocks, variant, y,
                                   sz.rows_max, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// The fused plan for small batches (include/moe.h, moe_grouped_ffn_fused)
// ---------------------------------------------------------------------------

// bf16 activations with bf16 or fp8 weights, no FP8 activation path and no shared
// experts
static moe_status fused_supported(const moe_problem* p) {
  if (p->act_dtype != MOE_BF16 || (p->weight_dtype != MOE_BF16 && p->weight_dtype != MOE_FP8_E4M3))
    return MOE_ERR_UNSUPPORTED;
  if (p->act_quant || p->shared_experts) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status moe_fused_workspace_bytes(const moe_problem* p, int64_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  st = fused_supported(p);
  if (st != MOE_OK) return st;
  *bytes = fused_ws_bytes(*p);
  return MOE_OK;
}

moe_status moe_grouped_ffn_fused(const moe_problem* p, const void* x, const void* w1,
                                 const void* w3, const void* w2, const float* s1, const float* s3,
                                 const float* s2, const int32_t* sorted_slots,
                                 const int32_t* block_expert, const int32_t* num_blocks,
                                 const int32_t* variant, void* fused_ws, size_t fused_ws_bytes_,
                                 void* stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  st = fused_supported(p);
  if (st != MOE_OK) return st;
  const bool fp8 = p->weight_dtype == MOE_FP8_E4M3;
  if (!x || !w1 || !w3 || !w2 || !sorted_slots || !block_expert || !num_blocks || !variant ||
      !fused_ws || (fp8 && (!s1 || !s3 || !s2)))
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w3, 16) || !aligned(w2, 16) ||
      !aligned(fused_ws, 256) || (fp8 && (!aligned(s1, 4) || !aligned(s3, 4) || !aligned(s2, 4))))
    return MOE_ERR_INVALID_ARG;
  if ((int64_t)fused_ws_bytes_ < fused_ws_bytes(*p)) return MOE_ERR_WORKSPACE;
  hipError_t err;
  const int cus = num_cus_current(&err);
  if (err != hipSuccess || cus <= 0) return MOE_ERR_HIP;
  return hip_status(launch_fused_ffn(*p, x, w1, w3, w2, fp8 ? s1 : nullptr, fp8 ? s3 : nullptr,
                                     fp8 ? s2 : nullptr, sorted_slots, block_expert, num_blocks,
                                     variant, fused_ws, cus, rows_max_of(p), (hipStream_t)stream));
}

moe_status moe_combine_fused(const moe_problem* p, const void* fused_ws, const int32_t* slot_pos,
                             const float* topk_w, void* y, void* stream) {
  moe_status st = validate(p);
  if (st != MOE_OK) return st;
  st = fused_supported(p);
  if (st != MOE_OK) return st;
  if (!fused_ws || !slot_pos || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned(fused_ws, 256) || !aligned(y, 16) || !aligned(topk_w, 4) || !aligned(slot_pos, 4))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine_fused(*p, fused_ws, slot_pos, topk_w, y, (hipStream_t)stream));
}

}  // extern "C"
