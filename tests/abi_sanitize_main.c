/*
 * abi_sanitize_main.c -- host-side checks of libmoe's C ABI for a build whose host
 * code runs under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitizers.py builds the library's API translation unit with the
 * host sanitizers and links this driver against it).
 *
 * Every call here returns from host validation before any kernel would be
 * enqueued, so the run needs no GPU: null pointers, bad shapes and dtypes,
 * misalignment, a too-small workspace, every query.  The device pointers passed
 * are never dereferenced on the host (they are placeholders), which is part of
 * what the sanitizers check.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../include/moe.h"

static int failures = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                 \
    const int got_ = (int)(call);                                                      \
    if (got_ != (int)(want)) {                                                         \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, \
              (int)(want));                                                            \
      ++failures;                                                                      \
    }                                                                                  \
  } while (0)

static moe_problem prob(int B, int H, int I, int E, int k, int act, int wt) {
  moe_problem p;
  memset(&p, 0, sizeof p);
  p.tokens = B;
  p.hidden = H;
  p.inter = I;
  p.num_experts = E;
  p.expert_begin = 0;
  p.local_experts = E;
  p.top_k = k;
  p.act_dtype = act;
  p.weight_dtype = wt;
  p.renormalize = 1;
  return p;
}

int main(void) {
  /* placeholder device addresses: aligned, never read by the host */
  void* D = (void*)(uintptr_t)0x10000;
  void* Dm = (void*)(uintptr_t)0x10004; /* misaligned for 16-byte operands */
  moe_sizes sz;
  int32_t info[MOE_VARIANT_FIELDS];

  EXPECT(moe_abi_version() > 0, 1);
  const int V = moe_num_variants();
  EXPECT(V >= 1, 1);
  for (int v = 0; v < V; ++v) EXPECT(moe_variant_info(v, info), MOE_OK);
  EXPECT(moe_variant_info(-1, info), MOE_ERR_INVALID_ARG);
  EXPECT(moe_variant_info(V, info), MOE_ERR_INVALID_ARG);
  EXPECT(moe_variant_info(0, NULL), MOE_ERR_INVALID_ARG);

  moe_problem ok = prob(64, 128, 256, 8, 2, MOE_F32, MOE_F32);
  EXPECT(moe_query_sizes(&ok, &sz), MOE_OK);
  EXPECT(sz.rows_max > 0 && sz.workspace_bytes > sz.rows_max, 1);
  EXPECT(moe_query_sizes(NULL, &sz), MOE_ERR_INVALID_ARG);
  EXPECT(moe_query_sizes(&ok, NULL), MOE_ERR_INVALID_ARG);

  /* shapes, dtypes and ranges validation refuses */
  moe_problem bad = ok;
  bad.tokens = 0;
  EXPECT(moe_query_sizes(&bad, &sz), MOE_ERR_INVALID_ARG);
  bad = ok;
  bad.hidden = 100;
  EXPECT(moe_query_sizes(&bad, &sz), MOE_ERR_INVALID_ARG);
  bad = ok;
  bad.top_k = 9;
  EXPECT(moe_query_sizes(&bad, &sz), MOE_ERR_INVALID_ARG);
  bad = ok;
  bad.expert_begin = 4;
  bad.local_experts = 5;
  EXPECT(moe_query_sizes(&bad, &sz), MOE_ERR_INVALID_ARG);
  bad = ok;
  bad.act_dtype = MOE_BF16;
  EXPECT(moe_query_sizes(&bad, &sz), MOE_ERR_UNSUPPORTED);
  bad = ok;
  bad.act_quant = 1;
  EXPECT(moe_query_sizes(&bad, &sz), MOE_ERR_UNSUPPORTED);
  bad = ok;
  bad.act_dtype = 7;
  EXPECT(moe_query_sizes(&bad, &sz), MOE_ERR_INVALID_ARG);
  bad = ok;
  bad.shared_experts = 99;
  EXPECT(moe_query_sizes(&bad, &sz), MOE_ERR_INVALID_ARG);
  bad = prob(1 << 20, 7168, 2048, 1024, 8, MOE_BF16, MOE_BF16);
  EXPECT(moe_query_sizes(&bad, &sz), MOE_ERR_UNSUPPORTED);

  /* every compute call: null pointers, misalignment, too small a workspace */
  EXPECT(moe_route_topk(&ok, NULL, D, D, D, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_route_topk(&bad, D, D, D, D, NULL), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_select_config(&ok, D, NULL, D, NULL, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_align_sort(&ok, D, D, NULL, D, D, D, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_route_select_align(&ok, D, D, D, D, D, D, D, NULL, D, D, D, NULL),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_grouped_ffn(&ok, D, D, D, D, NULL, NULL, NULL, D, D, D, D, D, D, 16, NULL),
         MOE_ERR_WORKSPACE);
  EXPECT(moe_grouped_ffn(&ok, Dm, D, D, D, NULL, NULL, NULL, D, D, D, D, D, D, 1ull << 40, NULL),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_grouped_ffn(&ok, D, D, D, D, NULL, NULL, NULL, D, D, D, D, D, Dm, 1ull << 40, NULL),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_grouped_gate_up(&ok, D, NULL, D, NULL, NULL, D, D, D, D, D, 1ull << 40, NULL),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_grouped_down(&ok, D, NULL, D, D, D, D, NULL, D, 1ull << 40, NULL),
         MOE_ERR_INVALID_ARG);
  moe_problem f8 = prob(64, 256, 256, 8, 2, MOE_BF16, MOE_FP8_E4M3);
  EXPECT(moe_grouped_ffn(&f8, D, D, D, D, NULL, D, D, D, D, D, D, D, D, 1ull << 40, NULL),
         MOE_ERR_INVALID_ARG); /* fp8 weights need their scales */
  EXPECT(moe_quant_act(&f8, D, D, D, NULL), MOE_ERR_INVALID_ARG); /* act_quant 0 */
  EXPECT(moe_combine(&ok, D, D, D, NULL, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_combine(&ok, Dm, D, D, D, NULL), MOE_ERR_INVALID_ARG);
  moe_problem sh = ok;
  sh.shared_experts = 1;
  EXPECT(moe_combine(&sh, D, D, D, D, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_combine_shared(&ok, D, D, D, D, D, D, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_cost_constants(&ok, NULL, NULL, NULL, NULL, NULL), MOE_ERR_INVALID_ARG);

  /* the fused small-batch plan */
  moe_problem fb = prob(3, 384, 256, 8, 2, MOE_BF16, MOE_BF16);
  int64_t fws = 0;
  EXPECT(moe_fused_workspace_bytes(&fb, &fws), MOE_OK);
  if (fws != 256 + 4ll * (256 / 32) * 3 * 2 * 384) {
    fprintf(stderr, "moe_fused_workspace_bytes: %lld\n", (long long)fws);
    ++failures;
  }
  EXPECT(moe_fused_workspace_bytes(&ok, &fws), MOE_ERR_UNSUPPORTED); /* fp32 */
  EXPECT(moe_fused_workspace_bytes(&fb, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_grouped_ffn_fused(&fb, D, D, D, D, NULL, NULL, NULL, D, D, D, D, D, (size_t)fws - 1,
                               NULL),
         MOE_ERR_WORKSPACE);
  EXPECT(moe_grouped_ffn_fused(&fb, Dm, D, D, D, NULL, NULL, NULL, D, D, D, D, D, 1ull << 40, NULL),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_grouped_ffn_fused(&f8, D, D, D, D, NULL, NULL, NULL, D, D, D, D, D, 1ull << 40, NULL),
         MOE_ERR_INVALID_ARG); /* fp8 weights need their scales */
  EXPECT(moe_combine_fused(&fb, D, D, D, NULL, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_combine_fused(&ok, D, D, D, D, NULL), MOE_ERR_UNSUPPORTED);

  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("ABI sanitize run: all checks passed (%d configurations)\n", V);
  return 0;
}
