/*
 * moe.h -- C ABI of the routing-aware fused Mixture-of-Experts layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer (GC-MoE, arXiv 2611.04222, section 2.1, Eq. 1, routed-expert term):
 *     y_t = sum_{j in TopK(t)} g_{t,j} * W2^(j) * SwiGLU(W1^(j) x_t),
 * with SwiGLU(v) = silu(W1 v) * (W3 v): W1 is the gate and W3 the up projection
 * (GC-MoE stacks them as one 2I x H matrix), W2 the down projection.  It runs as
 * five stream-ordered calls:
 *
 *   moe_route_topk     top-k of the router logits, softmax weights, and the
 *                      per-local-expert token histogram n_e (RaMP, arXiv
 *                      2604.26039, sections 2.1 and 2.3; the counting half of
 *                      the selection kernel of section 3.2).
 *   moe_select_config  the on-GPU cost model: for every compiled tile
 *                      configuration c, t_c = th0 + th1 W_c + th2 T_c + th3 A
 *                      (RaMP section 3.1, Eq. 3) over the row-tiles T_c and waves
 *                      W_c of section 2.2, Eq. 1, then c* = argmin_c t_c (section
 *                      2.4, Eq. 2), written to device memory.
 *   moe_align_sort     the routed slots grouped by expert and padded into the
 *                      chosen configuration's tiles (RaMP section 3.2).
 *   moe_route_select_align  the three steps above fused into fewer launches.
 *   moe_grouped_ffn    the polymorphic grouped expert kernel: every compiled
 *                      configuration lives in one kernel that reads c* from device
 *                      memory (RaMP section 3.3); gate/up with fused SwiGLU, then
 *                      the down projection (also callable one phase at a time:
 *                      moe_grouped_gate_up, moe_grouped_down).
 *   moe_combine        y_t = sum_j g_{t,j} y_{t,j}, accumulated in fp32 in j order
 *                      (GC-MoE section 4, the combine role).
 *
 * Conventions for every call
 *   - All array arguments are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises, and never reads device memory from
 *     the host, so every call can be captured in a HIP graph (the captured-forward
 *     constraint of RaMP section 2.4).  `stream` is a hipStream_t (NULL = the
 *     default stream); work is enqueued on it and the call returns.
 *   - Host-side validation runs first; on any error nothing is enqueued and the
 *     status says why.  A failed launch returns MOE_ERR_HIP.
 *   - Data-dependent values (counts, the chosen configuration, the block count)
 *     stay in device memory and are only read by the kernels.
 *   - Layouts are row-major.  Activations x [B][H]; router logits [B][E];
 *     per-expert weights in nn.Linear order [out][in]: W1, W3 [E_loc][I][H],
 *     W2 [E_loc][H][I].  FP8 weights are OCP E4M3FN codes with one fp32 scale per
 *     128 x 128 block of each (out, in) matrix, w = q * s (the block-scaled FP8 of
 *     RaMP section 3.3): s1, s3 [E_loc][I/128][H/128], s2 [E_loc][H/128][I/128].
 *   - Supported dtype combinations (act/out, weights): (f32, f32), (bf16, bf16),
 *     (bf16, fp8_e4m3).  The intermediate h and the per-slot outputs y_slots use
 *     the activation dtype; accumulation is always fp32.
 *   - FP8 activation path (act_quant = 1, bf16 x with fp8 weights only): the
 *     library quantizes x to E4M3FN per token and per 128-column group
 *     (moe_quant_act) and runs the gate/up GEMM with fp8 x fp8 matrix
 *     instructions, applying the activation and weight block scales to each
 *     128-deep partial sum (RaMP section 3.3 and appendix A.8: FP8 GEMMs with
 *     128 x 128 block scaling as used by DeepSeek-V3).  h stays bf16 and the down
 *     GEMM is unchanged.  act_quant = 2 also quantizes h (bf16, as the gate/up
 *     GEMM stores it) the same way, per slot row and 128-column group, at the
 *     start of the down phase, and runs the down GEMM on fp8 x fp8 too (RaMP
 *     appendix A.8 quantizes the gated activation to FP8 before the down
 *     projection).
 *   - Concurrent calls must not share one workspace or output buffer.
 *   - Shared experts (shared_experts > 0): after the routed row-blocks of the
 *     chosen configuration come, for each shared expert i, ceil(B / BLOCK_M)
 *     row-blocks holding tokens 0..B-1 in order; their rows of h and y_slots
 *     follow the routed rows.  The configuration choice counts them (each shared
 *     expert adds ceil(B / b) row-tiles and one active expert); the sort and the
 *     inverse map cover the routed slots only; moe_combine_shared adds lane k.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment, bad range   */
  MOE_ERR_UNSUPPORTED = -2, /* valid but not built: dtype mix, shape limits      */
  MOE_ERR_WORKSPACE = -3,   /* workspace smaller than moe_query_sizes() asks     */
  MOE_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed        */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* The device status word.  Host validation cannot see values that live in device
 * memory (the chosen configuration, the row-block count), so the grouped FFN
 * checks them on the device and reports what it found in the int32 at byte
 * offset MOE_DEVICE_STATUS_OFFSET of its workspace: 0 (MOE_DEV_OK) when both were
 * valid, else one of the codes below.  Every grouped-FFN launch rewrites it
 * (workgroup 0, once per launch), so after a call it describes that call's
 * inputs; the caller reads it with an ordinary device-to-host copy when it wants
 * to (the library itself never does).  What the kernels do on such inputs:
 *   MOE_DEV_BAD_VARIANT  *variant outside [0, V): no tile runs, y_slots and h are
 *                        not written (moe_align_sort has already written
 *                        num_blocks = 0 and slot_pos = -1 for such a variant, so
 *                        moe_combine then writes zeros);
 *   MOE_DEV_BAD_BLOCKS   *num_blocks < 0, or more row-blocks (shared experts'
 *                        included) than rows_max holds: only the row-blocks that
 *                        fit are computed. */
#define MOE_DEVICE_STATUS_OFFSET 0
#define MOE_DEV_OK 0
#define MOE_DEV_BAD_VARIANT 1
#define MOE_DEV_BAD_BLOCKS 2

/* The problem statement shared by every call (B tokens of H hidden activations,
 * E experts of intermediate size I, top-k routing; this GPU holds the contiguous
 * expert block [expert_begin, expert_begin + local_experts), as under expert
 * parallelism in RaMP section 2.1; a single GPU with all experts has
 * expert_begin = 0, local_experts = E). */
typedef struct moe_problem {
  int32_t tokens;        /* B >= 1                                              */
  int32_t hidden;        /* H: multiple of 128                                  */
  int32_t inter;         /* I: multiple of 128                                  */
  int32_t num_experts;   /* E, 1 <= E <= 4096                                   */
  int32_t expert_begin;  /* e0 >= 0                                             */
  int32_t local_experts; /* E_loc >= 1, e0 + E_loc <= E, E_loc <= 1024          */
  int32_t top_k;         /* k, 1 <= k <= min(E, 32)                             */
  int32_t act_dtype;     /* moe_dtype of x, h, y_slots and y: MOE_F32/MOE_BF16  */
  int32_t weight_dtype;  /* moe_dtype of W1, W3, W2                             */
  int32_t renormalize;   /* 1: softmax over the k chosen logits (default);
                            0: those experts' values of the softmax over all E  */
  int32_t act_quant;     /* 0: none (default); 1: x in FP8 for the gate/up GEMM;
                            2: x and h in FP8 for both GEMMs (see above; needs
                            act_dtype MOE_BF16, weight_dtype MOE_FP8_E4M3)      */
  int32_t shared_experts; /* S_sh, 0..8: experts every token goes through with
                            weight 1, fused into the same grouped FFN launches
                            (GC-MoE section 4: shared experts see every local
                            token, need no dispatch, and their output is one more
                            lane of the combine).  Their weights follow the local
                            experts' in W1, W3, W2 (and s1, s3, s2): those arrays
                            hold E_loc + S_sh experts.                          */
  const void* packed_weights; /* NULL (default), or a copy of W1, W3 and W2 that
                            moe_pack_wide wrote for this problem's shapes (device
                            memory, 256-byte aligned, owned by the caller, not
                            modified by any call).  When set, the wide
                            configuration's bf16 tiles read their weights from it
                            instead of W1, W3, W2; every other configuration
                            reads W1, W3, W2 as always, so those stay required.
                            Only for act_dtype = weight_dtype = MOE_BF16
                            (MOE_ERR_INVALID_ARG otherwise).                    */
} moe_problem;

/* Buffer sizes a caller must provide for one problem. */
typedef struct moe_sizes {
  int64_t rows_max;        /* capacity (elements) of sorted_slots; rows of y_slots */
  int64_t blocks_max;      /* capacity (elements) of block_expert                  */
  int64_t y_slots_bytes;   /* rows_max * H * sizeof(act)                           */
  int64_t workspace_bytes; /* grouped_ffn workspace: a 256-byte header (the device
                              status word first), h, (act_quant: x codes and
                              scales; 2: h codes and scales), partial tiles         */
  int64_t align_ws_bytes;  /* reserved, 0 in this version                          */
} moe_sizes;

/* ---- queries ------------------------------------------------------------- */

/* Version of this ABI (bumped on any incompatible change). */
int32_t moe_abi_version(void);

/* Shape limits (MOE_ERR_UNSUPPORTED beyond them): B * k < 2^30; the grouped
 * FFN reads x (B * H), h (rows_max * I) and one expert's weight matrix (I * H)
 * through 32-bit buffer offsets, so each of these is below 2^31 bytes, and
 * rows_max * max(H, I) elements of y_slots are below 2^31 bytes too; the
 * alignment step's tables fit one workgroup's LDS. */

/* Fills *out for problem *p.  Errors: MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED
 * with the same rules as the compute calls. */
moe_status moe_query_sizes(const moe_problem* p, moe_sizes* out);

/* Number V of tile configurations compiled into the polymorphic kernel. */
int32_t moe_num_variants(void);

/* Static description of configuration v, out[0..MOE_VARIANT_FIELDS-1]:
 *   [0] BLOCK_M  token rows per tile (b_c of RaMP Eq. 1)
 *   [1] BLOCK_N of the gate/up phase (output columns of W1 and of W3 per tile)
 *   [2] BLOCK_N of the down phase
 *   [3] BLOCK_K  reduction depth per pipeline stage for bf16 operands (the fp32
 *                problem uses half of it; fp8 weights are staged as bf16; in the
 *                wide class the fp32 and fp8 tiles stage twice the bytes)
 *   [4] waves along M, [5] waves along N, [6] waves splitting K inside a tile
 *       (of the bf16 tiles: the wide class's fp32 and fp8 tiles run twice the
 *       waves along N)
 *   [7] split-K of the down phase across tiles (1 = none)
 *   [8] 1 if weights are read with non-temporal (streaming) loads, 0 if cached
 *   [9] workgroups per compute unit of its persistent launch (its occupancy
 *       class: 2 for the streaming class, 1 for the wide class)
 *   [10] threads per workgroup of the bf16 tiles, 64 x [4] x [5] x [6]
 * Errors: MOE_ERR_INVALID_ARG for v outside [0, V) or out == NULL. */
#define MOE_VARIANT_FIELDS 11
moe_status moe_variant_info(int32_t v, int32_t* out);

/* The cost-model constants moe_select_config uses for problem *p on the current
 * HIP device, per configuration v (arrays of V int32, host memory):
 *   b[v]  = BLOCK_M;  q1[v] = ceil(I / BLOCK_N1), q2[v] = ceil(H / BLOCK_N2) * split_k,
 *   the tiles of one row-block in each phase (q_c of RaMP Eq. 1, summed over the
 *   two phases); S1[v], S2[v] = tiles resident on the GPU at once in each phase
 *   = the persistent grid of v's class, min(compute units * workgroups per CU,
 *   512) workgroups (S_c of RaMP Eq. 1).
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP. */
moe_status moe_cost_constants(const moe_problem* p, int32_t* b, int32_t* q1, int32_t* q2,
                              int32_t* S1, int32_t* S2);

/* ---- the five steps ------------------------------------------------------- */

/* Step 1: top-k routing and histogram (RaMP 2.1, 2.3, 3.2).
 *   logits   f32 [B][E]                      in
 *   topk_ids i32 [B][k]  global expert ids   out, descending logit; equal logits
 *                        go to the lower expert index and -0 equals +0
 *   topk_w   f32 [B][k]                      out, softmax weights (see renormalize)
 *   counts   i32 [E_loc]                     out, n_e = slots routed to local e
 * NaN logits are outside the contract. */
moe_status moe_route_topk(const moe_problem* p, const float* logits, int32_t* topk_ids,
                          float* topk_w, int32_t* counts, void* stream);

/* Step 2: choose the configuration (RaMP 3.1 Eq. 3, 3.2, 2.4 Eq. 2).
 *   counts  i32 [E_loc]        in (from moe_route_topk)
 *   theta   f32 [V][4]         in, th0..th3 per configuration (fit offline)
 *   variant i32 [1]            out, argmin_v t_v (first index on ties)
 *   t_hat   f32 [V] or NULL    out, the predictions (diagnostics)
 * t_v = fmaf(th3, A, fmaf(th2, T, fmaf(th1, W, th0))) in fp32 with
 * T = (q1 + q2) * sum_e ceil(n_e / b), W = ceil(q1 rt / S1) + ceil(q2 rt / S2),
 * rt = sum_e ceil(n_e / b), A = #{e : n_e > 0}, constants of moe_cost_constants. */
moe_status moe_select_config(const moe_problem* p, const int32_t* counts, const float* theta,
                             int32_t* variant, float* t_hat, void* stream);

/* Step 3: group and pad (RaMP 3.2).  With b = BLOCK_M of *variant:
 *   sorted_slots i32 [rows_max]  out; rows [0, R): for local expert e = 0..E_loc-1
 *                the slots s = t*k + j routed to e in ascending s, then -1 up to a
 *                multiple of b; R = num_blocks * b.  Rows >= R are not written.
 *   block_expert i32 [blocks_max] out; local expert of row-block i < num_blocks
 *   num_blocks   i32 [1]          out
 *   slot_pos     i32 [B*k]        out; row of slot s, or -1 if s is not local
 * A *variant outside [0, V) yields num_blocks = 0 and slot_pos = -1 everywhere. */
moe_status moe_align_sort(const moe_problem* p, const int32_t* topk_ids, const int32_t* variant,
                          int32_t* sorted_slots, int32_t* block_expert, int32_t* num_blocks,
                          int32_t* slot_pos, void* stream);

/* Steps 1-3 fused: exactly moe_route_topk, then moe_select_config (when theta is
 * not NULL), then moe_align_sort, with the same arguments and bit-identical
 * outputs, in fewer launches.  RaMP section 3.2 describes one selection kernel
 * that counts, chooses and lays out the tiles; here a batch that one workgroup
 * routes (B <= 4 * (1024 / L), L the lanes per token: the smallest power of two
 * >= E up to 64) runs in a single one-workgroup launch, a larger one as the
 * routing launch(es) followed by one select-and-align launch.  theta NULL: no
 * selection; the configuration already in *variant is used and t_hat is not
 * written (t_hat may be NULL in any case).  Errors: as the three calls. */
moe_status moe_route_select_align(const moe_problem* p, const float* logits, const float* theta,
                                  int32_t* topk_ids, float* topk_w, int32_t* counts,
                                  int32_t* variant, float* t_hat, int32_t* sorted_slots,
                                  int32_t* block_expert, int32_t* num_blocks, int32_t* slot_pos,
                                  void* stream);

/* FP8 activation quantization (the first launch of the gate/up phase when
 * act_quant = 1; callable alone for tests).  For every token t and group g of 128
 * hidden columns of bf16 x [B][H]:
 *   amax = max_i |x[t][128g + i]|,  xs[t][g] = amax / 448 (fp32 division),
 *   xq[t][128g + i] = E4M3FN code nearest to clamp(x / xs, -448, 448) (fp32
 *                     division; ties to the even code; a negative value that
 *                     rounds to zero gives 0x80),
 * and a group of zeros gets xs = 0 and codes 0x00.  x = q * s then holds to
 * within half a code step.  xq uint8 [B][H], xs f32 [B][H/128], device memory.
 * Requires act_quant = 1 or 2; errors as the other calls. */
moe_status moe_quant_act(const moe_problem* p, const void* x, uint8_t* xq, float* xs,
                         void* stream);

/* Step 4: grouped expert FFN (RaMP 3.3 and A.8; GC-MoE 2.1 Eq. 1).  For every
 * row r < R that holds a slot (sorted_slots[r] >= 0):
 *   h[r]       = silu(x[t] W1_e^T) * (x[t] W3_e^T)   (t = sorted_slots[r] / k)
 *   y_slots[r] = h[r] W2_e^T                          (e = block_expert[r / b])
 * Padding rows are neither read nor written.  x is [B][H] (act dtype); s1/s3/s2
 * are the fp8 block scales (NULL unless weight_dtype is MOE_FP8_E4M3).  y_slots
 * [rows_max][H] (act dtype).  workspace: >= workspace_bytes, 256-byte aligned;
 * holds h and the fp32 partial sums of the tiles that a phase's last round splits
 * across workgroups.  The call enqueues, for the gate/up phase and then the down
 * phase (moe_grouped_gate_up followed by moe_grouped_down), two launches of
 * persistent polymorphic kernels, one per occupancy class of the compiled
 * configurations (2 workgroups of 256 threads per CU; 1 workgroup per CU, of 256
 * threads for bf16 and 512 for fp32 and fp8): each runs the
 * chosen configuration if it belongs to its class, and the second also adds the
 * partial sums of the tiles the first class split.  With bf16 weights and
 * activations the down phase adds a third launch when the problem's row-block
 * bound lets the one-per-CU configuration split its last round (more tiles than
 * one round of its grid): it adds that configuration's split tiles.  Every launch
 * reads *variant and *num_blocks from device memory, so every compiled
 * configuration runs under one fixed launch shape. */
moe_status moe_grouped_ffn(const moe_problem* p, const void* x, const void* w1, const void* w3,
                           const void* w2, const float* s1, const float* s3, const float* s2,
                           const int32_t* sorted_slots, const int32_t* block_expert,
                           const int32_t* num_blocks, const int32_t* variant, void* y_slots,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Step 4 for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * moe_grouped_ffn, with the same arguments apart from the workspace, which here is
 * an array the library owns on each GPU (moe_noalloc_workspace_limit() bytes,
 * 256 MiB, reserved when the library is loaded on that GPU and held until the
 * process ends).  The call allocates and frees nothing.  Its outputs are the
 * bits moe_grouped_ffn writes for the same inputs.
 *   - Problems whose moe_query_sizes().workspace_bytes exceed the limit get
 *     MOE_ERR_WORKSPACE, with nothing enqueued.
 *   - Every call on one GPU uses that GPU's one array and overwrites what the
 *     previous call left there; nothing in it needs to start at zero.  Calls
 *     that overlap in time on one GPU (on different streams, or from several
 *     host threads) race on it: serialize them.
 *   - The device status word of such a call is at MOE_DEVICE_STATUS_OFFSET of
 *     the library's array and is not readable through this ABI.
 * Errors: as moe_grouped_ffn; MOE_ERR_HIP if the array's device address cannot
 * be obtained on the current device. */
moe_status moe_grouped_ffn_noalloc(const moe_problem* p, const void* x, const void* w1,
                                   const void* w3, const void* w2, const float* s1,
                                   const float* s3, const float* s2, const int32_t* sorted_slots,
                                   const int32_t* block_expert, const int32_t* num_blocks,
                                   const int32_t* variant, void* y_slots, void* stream);

/* Size in bytes of the per-GPU array moe_grouped_ffn_noalloc works in. */
int64_t moe_noalloc_workspace_limit(void);

/* Weight prepack for the wide configuration (GC-MoE, arXiv 2611.04222, section
 * 4: a weight transform, run once per weight set on the caller's stream, that
 * makes each tile's reduction blocks contiguous and interleaves gate and up;
 * RaMP appendix A.8 loads gate and up weights interleaved).  The copy holds, for
 * every expert e (E_loc + S_sh of them), in this order:
 *   gate/up: for each column tile n of ceil(I / 128), for each 32-deep block kb
 *     of H: 256 rows of 64 bytes, rows 0-127 = W1_e[128 n + r][32 kb .. 32 kb + 31],
 *     rows 128-255 = W3_e of the same rows (rows past I are zeros);
 *   then down, for every expert: for each column tile n of ceil(H / 256), for each
 *     32-deep block kb of I: 256 rows of 64 bytes, W2_e[256 n + r][32 kb ..]
 *     (rows past H zeros).
 * Each 16 KiB block is one pipeline stage of that configuration's tile, so a
 * stage's weight loads read 16 KiB of consecutive bytes instead of 64 bytes of
 * each of 256 rows.
 * moe_pack_wide_bytes: *bytes = the copy's size (2 * E * ceil(I/128) * 128 * H + E *
 * ceil(H/256) * 256 * I bf16 values).  moe_pack_wide: writes the copy to packed
 * (device, 256-byte aligned, *bytes) from W1, W3, W2 ([E][I][H], [E][I][H],
 * [E][H][I] bf16, device); enqueued on stream, asynchronous.  Errors:
 * MOE_ERR_INVALID_ARG (NULL pointers, misalignment, p not bf16 or with
 * packed_weights set), MOE_ERR_UNSUPPORTED, MOE_ERR_HIP. */
moe_status moe_pack_wide_bytes(const moe_problem* p, int64_t* bytes);
moe_status moe_pack_wide(const moe_problem* p, const void* w1, const void* w3, const void* w2,
                         void* packed, void* stream);

/* Step 4a alone: the grouped gate/up GEMM with the fused SwiGLU, writing h into
 * workspace (as moe_grouped_ffn's first launch; with act_quant = 1 it is preceded
 * by moe_quant_act of x into the workspace).  Arguments and errors as for
 * moe_grouped_ffn; w2, s2 and y_slots are not used. */
moe_status moe_grouped_gate_up(const moe_problem* p, const void* x, const void* w1,
                               const void* w3, const float* s1, const float* s3,
                               const int32_t* sorted_slots, const int32_t* block_expert,
                               const int32_t* num_blocks, const int32_t* variant, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Step 4b alone: the grouped down GEMM, y_slots[r] = h[r] W2_e^T with h read from
 * workspace (written by moe_grouped_gate_up for the same grouping and variant;
 * with act_quant = 2 the rows of h that hold a slot are first quantized in the
 * workspace, as moe_quant_act does for x).
 * Arguments and errors as for moe_grouped_ffn; x, w1, w3, s1 and s3 are not
 * used. */
moe_status moe_grouped_down(const moe_problem* p, const void* w2, const float* s2,
                            const int32_t* sorted_slots, const int32_t* block_expert,
                            const int32_t* num_blocks, const int32_t* variant, void* y_slots,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Step 5 with shared experts: as moe_combine, then, after the k routed lanes,
 * y_t += y_slots[(num_blocks + i * ceil(B / b)) * b + t] for i = 0..S_sh-1, with
 * weight 1 (b = BLOCK_M of *variant): the shared experts' lanes of the combine
 * (GC-MoE section 4).  num_blocks and variant are the device values the sort
 * wrote.  Errors: as moe_combine; MOE_ERR_INVALID_ARG for shared_experts = 0. */
moe_status moe_combine_shared(const moe_problem* p, const void* y_slots, const int32_t* slot_pos,
                              const float* topk_w, const int32_t* num_blocks,
                              const int32_t* variant, void* y, void* stream);

/* Step 5: combine (GC-MoE 2.1 Eq. 1; the slot-order reduction of its combine
 * role).  Problems with shared experts use moe_combine_shared instead
 * (MOE_ERR_INVALID_ARG here).  y [B][H] (act dtype) = sum over j = 0..k-1 with slot_pos[t*k+j] >= 0 of
 * topk_w[t][j] * y_slots[slot_pos[t*k+j]], in fp32, rounded to nearest even once;
 * tokens with no local slot get zeros. */
moe_status moe_combine(const moe_problem* p, const void* y_slots, const int32_t* slot_pos,
                       const float* topk_w, void* y, void* stream);

/* The fused plan for small batches (RaMP appendix A.8, "Fusion": each tile runs
 * the up-projection, the gated activation and the down-projection in turn, and
 * adds its down-projection result into the layer's output).  It replaces steps 4
 * and 5 (moe_grouped_ffn, moe_combine) with one FFN launch and one combine launch;
 * steps 1-3 are unchanged.  A tile is one row-block of the alignment (BLOCK_M of
 * *variant) times one slice of 32 columns of I:
 *   h_j[r]       = bf16(silu(x[t] W1_e[slice j]^T) * (x[t] W3_e[slice j]^T))
 *   part[j][s]   = h_j[r] W2_e[:, slice j]^T              (fp32)
 * for every row r that holds slot s = sorted_slots[r] (t = s / k, e =
 * block_expert[r / b]); the combine then writes
 *   y[t] = sum over i = 0..k-1 with slot_pos[t*k+i] >= 0, and over j, of
 *          topk_w[t][i] * part[j][t*k+i]
 * in fp32 in a fixed order (pair p = i * (I/32) + j goes to lane p mod 32; each
 * of the 32 lanes adds its pairs in ascending p, then the lanes are added in
 * order), rounded to bf16 once.  No atomics, so the result is deterministic.  Compared with the
 * grouped plan, the sum over I is added per 32-column slice and nothing is
 * rounded to bf16 before the combine (there is no y_slots).
 * Where it pays: each tile streams its slice of W1, W3 and W2 once, and the
 * partial rows add 4 * B * k * H * I / 32 bytes, written once and read once; at
 * a few token rows per expert that is a small share of the weight bytes, and the
 * FFN is one launch instead of four.  The caller chooses the plan by batch size.
 * Supported problems: bf16 activations with bf16 or fp8 weights, act_quant = 0,
 * no shared experts (else MOE_ERR_UNSUPPORTED).  With packed_weights set (bf16
 * problems, moe_pack_wide) the FFN reads the weights from the packed copy, whose
 * blocks give each fragment load 1 KiB of consecutive bytes (W1, W3 and W2 must
 * still be passed); the result is bit-identical to reading W1, W3, W2.
 * moe_fused_workspace_bytes: *bytes = 256 + 4 * (I / 32) * B * k * H, the size
 *   of fused_ws: a 256-byte header whose int32 at MOE_DEVICE_STATUS_OFFSET is the
 *   device status word (as for moe_grouped_ffn; written by every fused FFN
 *   launch), then part [I/32][B*k][H] fp32.  Only the rows of local slots are
 *   written; nothing needs to start at zero.
 * moe_grouped_ffn_fused: x [B][H] bf16, weights and scales as moe_grouped_ffn,
 *   sorted_slots / block_expert / num_blocks / variant from steps 1-3 (device);
 *   fused_ws device, 256-byte aligned, >= fused_ws_bytes bytes (else
 *   MOE_ERR_WORKSPACE).  One persistent launch of 256-thread workgroups.
 * moe_combine_fused: reads fused_ws after moe_grouped_ffn_fused on the same
 *   stream; y [B][H] bf16.  Tokens with no local slot get zeros, and so does
 *   every token when the status word is not MOE_DEV_OK.
 * Errors: MOE_ERR_INVALID_ARG (NULL pointers, misalignment), MOE_ERR_UNSUPPORTED,
 * MOE_ERR_WORKSPACE, MOE_ERR_HIP; all calls are asynchronous on stream. */
moe_status moe_fused_workspace_bytes(const moe_problem* p, int64_t* bytes);
moe_status moe_grouped_ffn_fused(const moe_problem* p, const void* x, const void* w1,
                                 const void* w3, const void* w2, const float* s1, const float* s3,
                                 const float* s2, const int32_t* sorted_slots,
                                 const int32_t* block_expert, const int32_t* num_blocks,
                                 const int32_t* variant, void* fused_ws, size_t fused_ws_bytes,
                                 void* stream);
moe_status moe_combine_fused(const moe_problem* p, const void* fused_ws, const int32_t* slot_pos,
                             const float* topk_w, void* y, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
