/*
 * sanitize_main.c -- a driver that runs every entry point of the CPU oracle
 * (moe_oracle.c) on small inputs, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py builds and runs it).
 *
 * TEST INFRASTRUCTURE ONLY, like the oracle itself.  Each call is followed by a
 * cheap invariant so that the run also fails on a wrong result, not only on an
 * out-of-bounds access or undefined behaviour: distinct top-k ids and weights
 * that sum to 1, counts that sum to the local slots, a bijective alignment, a
 * select index within range, round-tripping fp8 codes, finite FFN outputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's entry points (moe_oracle.c) */
int oracle_route_topk(int B, int E, int k, int renormalize, const float* logits, int32_t* ids,
                      double* w);
void oracle_counts(int B, int k, int e0, int E_loc, const int32_t* ids, int32_t* counts);
int oracle_select(int E_loc, const int32_t* counts, int V, const int32_t* b, const int32_t* q1,
                  const int32_t* q2, const int32_t* S1, const int32_t* S2, const float* theta,
                  float* t_hat, int32_t* feat);
int64_t oracle_align(int B, int k, int e0, int E_loc, const int32_t* ids, int b,
                     int32_t* sorted_slots, int64_t cap, int32_t* block_expert,
                     int32_t* num_blocks, int32_t* slot_pos);
int oracle_ffn_slots(int H, int I, const void* x, int xdt, const void* w1, const void* w3,
                     const void* w2, int wdt, const float* s1, const float* s3, const float* s2,
                     int n, const int32_t* tok, const int32_t* exp_local, double* y, int nthreads,
                     int hq);
int oracle_layer_tokens(int H, int I, int k, int e0, int E_loc, const void* x, int xdt,
                        const void* w1, const void* w3, const void* w2, int wdt, const float* s1,
                        const float* s3, const float* s2, const int32_t* ids, const double* w,
                        int n_tok, const int32_t* tokens, double* Y, int nthreads, int hq,
                        int n_shared);
void oracle_decode_fp8(const uint8_t* codes, int64_t n, double* out);
void oracle_decode_bf16(const uint16_t* bits, int64_t n, double* out);
int oracle_quant_act_e4m3(int B, int H, const uint16_t* x, uint8_t* q, float* s);
int oracle_e4m3_round(const float* v, int64_t n, uint8_t* q);

static int failures = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                  \
    }                                                              \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, uniform in [0, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}
static float nrand(float sd) { return (float)((urand() + urand() + urand() - 1.5) * 2.0 * sd); }

static uint16_t f32_to_bf16(float f) { /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static void test_route_align(int B, int E, int k, int e0, int E_loc, int b) {
  float* lg = malloc(sizeof(float) * B * E);
  int32_t* ids = malloc(sizeof(int32_t) * B * k);
  double* w = malloc(sizeof(double) * B * k);
  int32_t* cnt = malloc(sizeof(int32_t) * E_loc);
  for (int i = 0; i < B * E; ++i) lg[i] = (float)((int)(urand() * 7) - 3) * 0.5f; /* many ties */
  for (int renorm = 0; renorm < 2; ++renorm) {
    CHECK(oracle_route_topk(B, E, k, renorm, lg, ids, w) == 0);
    for (int t = 0; t < B; ++t) {
      double sw = 0;
      for (int j = 0; j < k; ++j) {
        sw += w[t * k + j];
        for (int i = 0; i < j; ++i) CHECK(ids[t * k + i] != ids[t * k + j]);
      }
      if (renorm) CHECK(fabs(sw - 1.0) < 1e-12);
    }
  }
  oracle_counts(B, k, e0, E_loc, ids, cnt);
  int64_t local = 0, tot = 0;
  for (int s = 0; s < B * k; ++s) local += ids[s] >= e0 && ids[s] < e0 + E_loc;
  for (int e = 0; e < E_loc; ++e) tot += cnt[e];
  CHECK(tot == local);
  const int64_t cap = (int64_t)B * k + (int64_t)E_loc * (b - 1);
  int32_t* ss = malloc(sizeof(int32_t) * (cap > 0 ? cap : 1));
  int32_t* be = malloc(sizeof(int32_t) * (cap / b + 1));
  int32_t* sp = malloc(sizeof(int32_t) * B * k);
  int32_t nb = -1;
  const int64_t R = oracle_align(B, k, e0, E_loc, ids, b, ss, cap, be, &nb, sp);
  CHECK(R >= 0 && R % b == 0 && nb == R / b);
  int64_t seen = 0;
  for (int64_t r = 0; r < R; ++r)
    if (ss[r] >= 0) {
      CHECK(sp[ss[r]] == r);
      ++seen;
    }
  CHECK(seen == local);
  /* too small a capacity is refused, not overrun */
  if (R > 0) CHECK(oracle_align(B, k, e0, E_loc, ids, b, ss, R - 1, be, &nb, sp) == -1);
  free(lg);
  free(ids);
  free(w);
  free(cnt);
  free(ss);
  free(be);
  free(sp);
}

static void test_select(void) {
  enum { V = 5, EL = 48 };
  int32_t cnt[EL], b[V] = {16, 32, 64, 128, 256}, q1[V], q2[V], S1[V], S2[V], feat[3 * V];
  float th[4 * V], t_hat[V];
  for (int e = 0; e < EL; ++e) cnt[e] = urand() < 0.3 ? 0 : (int32_t)(urand() * 900);
  for (int v = 0; v < V; ++v) {
    q1[v] = 2048 / b[v];
    q2[v] = 7168 / b[v];
    S1[v] = S2[v] = 512;
    for (int c = 0; c < 4; ++c) th[4 * v + c] = (float)(urand() * 10.0);
  }
  const int c = oracle_select(EL, cnt, V, b, q1, q2, S1, S2, th, t_hat, feat);
  CHECK(c >= 0 && c < V);
  for (int v = 0; v < V; ++v) CHECK(t_hat[c] <= t_hat[v]);
  b[2] = 0; /* invalid tile height: refused */
  CHECK(oracle_select(EL, cnt, V, b, q1, q2, S1, S2, th, t_hat, feat) == -1);
}

static void test_codecs(void) {
  uint8_t codes[256], q[256];
  double vals[256];
  float f[256];
  int n = 0;
  for (int c = 0; c < 256; ++c)
    if ((c & 0x7F) != 0x7F) codes[n++] = (uint8_t)c; /* finite codes */
  oracle_decode_fp8(codes, n, vals);
  for (int i = 0; i < n; ++i) f[i] = (float)vals[i];
  CHECK(oracle_e4m3_round(f, n, q) == 0);
  for (int i = 0; i < n; ++i) CHECK(q[i] == codes[i] || (vals[i] == 0.0 && (q[i] & 0x7F) == 0));
  float big = 500.0f;
  CHECK(oracle_e4m3_round(&big, 1, q) != 0);
  uint16_t bits[4] = {0x3F80, 0xBF80, 0x0000, 0x4049};
  double d[4];
  oracle_decode_bf16(bits, 4, d);
  CHECK(d[0] == 1.0 && d[1] == -1.0 && d[2] == 0.0);
  enum { B = 3, H = 256 };
  uint16_t x[B * H];
  uint8_t xq[B * H];
  float xs[B * (H / 128)];
  for (int i = 0; i < B * H; ++i) x[i] = f32_to_bf16(nrand(1.0f));
  for (int i = 0; i < 128; ++i) x[H + i] = 0; /* a group of zeros */
  CHECK(oracle_quant_act_e4m3(B, H, x, xq, xs) == 0);
  CHECK(xs[2] == 0.0f);
  CHECK(oracle_quant_act_e4m3(B, 200, x, xq, xs) != 0); /* H not a multiple of 128 */
}

/* a tiny layer in each weight dtype, with and without h quantization and shared
 * experts */
static void test_layer(int wdt, int hq, int n_shared) {
  enum { H = 256, I = 128, E = 4, K = 2, BT = 5 };
  const int El = E + n_shared;
  const size_t nw = (size_t)El * I * H;
  const size_t wsz = wdt == 0 ? 4 : (wdt == 1 ? 2 : 1);
  void* w1 = malloc(nw * wsz);
  void* w3 = malloc(nw * wsz);
  void* w2 = malloc(nw * wsz);
  float* s1 = malloc(sizeof(float) * El * (I / 128) * (H / 128));
  float* s3 = malloc(sizeof(float) * El * (I / 128) * (H / 128));
  float* s2 = malloc(sizeof(float) * El * (H / 128) * (I / 128));
  for (size_t i = 0; i < nw; ++i) {
    for (int m = 0; m < 3; ++m) {
      void* wm = m == 0 ? w1 : (m == 1 ? w3 : w2);
      const float v = nrand(0.05f);
      if (wdt == 0) ((float*)wm)[i] = v;
      else if (wdt == 1) ((uint16_t*)wm)[i] = f32_to_bf16(v);
      else ((uint8_t*)wm)[i] = (uint8_t)(urand() * 256) & 0xF7; /* no NaN codes */
    }
  }
  for (int i = 0; i < El * (I / 128) * (H / 128); ++i) s1[i] = s3[i] = s2[i] = 0.01f;
  float xf[BT * H];
  uint16_t xb[BT * H];
  for (int i = 0; i < BT * H; ++i) {
    xf[i] = nrand(1.0f);
    xb[i] = f32_to_bf16(xf[i]);
  }
  const void* x = wdt == 0 ? (const void*)xf : (const void*)xb;
  const int xdt = wdt == 0 ? 0 : 1;
  int32_t ids[BT * K];
  double w[BT * K];
  float lg[BT * E];
  for (int i = 0; i < BT * E; ++i) lg[i] = nrand(1.0f);
  CHECK(oracle_route_topk(BT, E, K, 1, lg, ids, w) == 0);
  int32_t toks[BT] = {0, 1, 2, 3, 4};
  double Y[BT * H];
  CHECK(oracle_layer_tokens(H, I, K, 0, E, x, xdt, w1, w3, w2, wdt, s1, s3, s2, ids, w, BT, toks,
                            Y, 2, hq, n_shared) == 0);
  for (int i = 0; i < BT * H; ++i) CHECK(isfinite(Y[i]));
  int32_t el[BT] = {0, 1, 2, 3, 0};
  double ys[BT * H];
  CHECK(oracle_ffn_slots(H, I, x, xdt, w1, w3, w2, wdt, s1, s3, s2, BT, toks, el, ys, 2, hq) == 0);
  for (int i = 0; i < BT * H; ++i) CHECK(isfinite(ys[i]));
  free(w1);
  free(w3);
  free(w2);
  free(s1);
  free(s3);
  free(s2);
}

int main(void) {
  test_route_align(7, 6, 3, 0, 6, 4);
  test_route_align(40, 128, 8, 32, 32, 16);
  test_route_align(1, 8, 8, 0, 8, 128);
  test_route_align(9, 384, 8, 336, 48, 64); /* the last expert block */
  test_select();
  test_codecs();
  for (int wdt = 0; wdt < 3; ++wdt) test_layer(wdt, 0, 0);
  test_layer(2, 1, 0);
  test_layer(1, 0, 2);
  test_layer(2, 1, 1);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle sanitize run: all checks passed\n");
  return 0;
}
