/*
 * moe_oracle.c -- plain, slow CPU oracle of the routing-aware fused-MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  The GPU library never links,
 * includes or calls it, and it shares no code, header, table or helper with the
 * GPU path: it has its own fp8/bf16 decoders, its own top-k, softmax, counting
 * sort and expert FFN.  All floating point is fp64 except the cost model, which
 * the selection step evaluates in fp32 by definition (both sides must take the
 * same integer decision in the same precision).
 *
 * What it computes, step by step (sources are the three pages on routing-aware
 * MoE kernels: RaMP arXiv 2604.26039, GC-MoE arXiv 2611.04222, "Decoding the
 * Skew" arXiv 2607.23099):
 *
 *  O1 route    - top-k of each token's router logits, weights = softmax over the
 *                k picks (RaMP 2.1: a router sends each token to k of E experts;
 *                GC-MoE 2.1 Eq. 1 weights each expert output by g_{t,j}).
 *  O2 counts   - n_e, the tokens per local expert (RaMP 2.3: the n_e sum to Bk).
 *  O3 select   - row-tiles T_c and waves W_c (RaMP 2.2 Eq. 1), active experts A,
 *                predicted time t_c = th0 + th1 W + th2 T + th3 A (RaMP 3.1 Eq. 3),
 *                argmin over the configurations (RaMP 2.4 Eq. 2).
 *  O4 align    - the local slots grouped by expert and padded to the chosen
 *                configuration's tile rows (RaMP 3.2), with a block->expert table.
 *  O5 ffn      - per routed slot, W2 * SwiGLU(W1 x) with SwiGLU = silu(gate)*up
 *                (GC-MoE 2.1 Eq. 1; RaMP 2.1 gated MLP).
 *  O6 combine  - y_t = sum_j g_{t,j} * y_{t,j}, in j order (GC-MoE 2.1 Eq. 1).
 *                With shared experts (GC-MoE 4: every token goes through them and
 *                their output is one more lane of the combine), after the k routed
 *                lanes y_t += FFN_{E_loc + i}(x_t) for each shared expert i, with
 *                weight 1; their weights follow the local experts' in W1, W3, W2.
 *  Q  act quant - the optional FP8 activation path: x quantized to E4M3FN per
 *                token and per group of 128 hidden columns with an fp32 scale
 *                (RaMP 3.3 and A.8: FP8 with 128 x 128 block scaling as used by
 *                DeepSeek-V3, whose activations are scaled per 1 x 128 group);
 *                the expert FFN then runs on the dequantized x = q * s.  With h
 *                quantization as well (RaMP A.8 quantizes the gated activation to
 *                FP8 before the down projection), h is rounded to bf16 (the
 *                intermediate precision) and quantized the same way, per slot row
 *                and 128-column group, and the down projection uses q * s.
 *
 * Readings of points the pages leave open (each stated where it is used):
 *  - top-k compares raw fp32 logits; equal logits go to the lower expert index
 *    and -0 equals +0 (IEEE ">" never replaces an equal earlier pick).
 *  - tokens inside one expert group keep ascending slot order s = t*k + j;
 *    padding rows hold -1; experts with no tokens get no tile.
 *  - T and W of a two-phase (gate/up, then down) configuration sum over phases;
 *    A is the number of local experts with n_e > 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2, ORC_F64 = 3 };

/* ---------------------------------------------------------------- decoders -- */

/* bf16 is the upper half of an IEEE binary32; the conversion to double is exact. */
static double orc_bf16_to_f64(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities,
 * S.1111.111 is NaN; exponent 0 encodes subnormals m/8 * 2^-6.  Largest 448. */
double oracle_fp8_e4m3fn_to_f64(uint8_t code) {
  int sign = code >> 7;
  int ex = (code >> 3) & 0xF;
  int man = code & 0x7;
  double v;
  if (ex == 0xF && man == 0x7) return NAN;
  if (ex == 0)
    v = ldexp((double)man, -9);
  else
    v = ldexp(1.0 + (double)man / 8.0, ex - 7);
  return sign ? -v : v;
}

void oracle_decode_fp8(const uint8_t* codes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_e4m3fn_to_f64(codes[i]);
}

void oracle_decode_bf16(const uint16_t* bits, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f64(bits[i]);
}

/* Element (r, c) of expert e's weight matrix of shape rows x cols, as the exact
 * value the layer uses: w = q * s for fp8 with one scale per 128x128 block. */
static double orc_weight(const void* w, int dt, const float* scale, int e, int rows, int cols,
                         int r, int c) {
  int64_t idx = ((int64_t)e * rows + r) * cols + c;
  if (dt == ORC_F32) return (double)((const float*)w)[idx];
  if (dt == ORC_BF16) return orc_bf16_to_f64(((const uint16_t*)w)[idx]);
  {
    int64_t sidx = ((int64_t)e * (rows / 128) + r / 128) * (cols / 128) + c / 128;
    return oracle_fp8_e4m3fn_to_f64(((const uint8_t*)w)[idx]) * (double)scale[sidx];
  }
}

static double orc_act(const void* x, int dt, int64_t idx) {
  if (dt == ORC_F32) return (double)((const float*)x)[idx];
  if (dt == ORC_F64) return ((const double*)x)[idx];
  return orc_bf16_to_f64(((const uint16_t*)x)[idx]);
}

/* ------------------------------------------------- Q: activation quantizer -- */

/* The E4M3FN code nearest to v, for |v| <= 448.  vals[c] is the value of code c
 * for c = 0..126 (the finite non-negative codes, increasing with c).  A value
 * halfway between two neighbouring codes takes the one whose code is even (the
 * round-to-nearest-even rule of IEEE conversions).  The sign bit is v's sign bit,
 * so a negative value that rounds to zero gives 0x80 (as an IEEE conversion keeps
 * the sign of a result that underflows to zero). */
static uint8_t orc_e4m3_nearest(float v, const double* vals) {
  const double a = fabs((double)v);
  int lo = 0, hi = 126;  /* invariant: vals[lo] <= a, answer in [lo, hi] */
  if (a >= vals[126]) {
    lo = 126;
  } else {
    while (hi - lo > 1) {  /* bisection for the largest lo with vals[lo] <= a */
      int mid = (lo + hi) / 2;
      if (vals[mid] <= a) lo = mid; else hi = mid;
    }
    {
      double dlo = a - vals[lo], dhi = vals[lo + 1] - a;
      if (dhi < dlo || (dhi == dlo && ((lo + 1) & 1) == 0)) lo = lo + 1;
    }
  }
  return (uint8_t)((signbit(v) ? 0x80 : 0x00) | lo);
}

/* Q: per token t and per group g of 128 hidden columns of bf16 x [B][H]:
 *   amax = max |x[t][128g + i]| (fp32, exact), s[t][g] = amax / 448 (fp32 division),
 *   q[t][128g + i] = the nearest E4M3FN code of min(max(x / s, -448), 448), with
 *   x / s an fp32 division, so that x is approximately q * s with the group's
 *   largest magnitude mapped onto 448, the largest E4M3FN value.  A group whose
 *   values are all zero gets s = 0 and codes 0x00.  Returns 0, or -1 for H not a
 *   multiple of 128. */
int oracle_quant_act_e4m3(int B, int H, const uint16_t* x, uint8_t* q, float* s) {
  double vals[127];
  if (B < 0 || H % 128) return -1;
  for (int c = 0; c <= 126; ++c) vals[c] = oracle_fp8_e4m3fn_to_f64((uint8_t)c);
  const int G = H / 128;
  for (int t = 0; t < B; ++t)
    for (int g = 0; g < G; ++g) {
      const uint16_t* xr = x + (int64_t)t * H + (int64_t)g * 128;
      uint8_t* qr = q + (int64_t)t * H + (int64_t)g * 128;
      float amax = 0.0f;
      for (int i = 0; i < 128; ++i) {
        float a = fabsf((float)orc_bf16_to_f64(xr[i]));
        if (a > amax) amax = a;
      }
      const float sc = amax / 448.0f;
      s[(int64_t)t * G + g] = sc;
      for (int i = 0; i < 128; ++i) {
        if (amax == 0.0f) {
          qr[i] = 0;
          continue;
        }
        float v = (float)orc_bf16_to_f64(xr[i]) / sc;
        if (v > 448.0f) v = 448.0f;
        if (v < -448.0f) v = -448.0f;
        qr[i] = orc_e4m3_nearest(v, vals);
      }
    }
  return 0;
}

/* h quantization of one row of n (a multiple of 128) values, in place: each value
 * rounded to bf16 (fp64 -> fp32 -> bf16, each to nearest even: the row is held in
 * fp32 and stored as bf16 before it is quantized), then Q on the bf16 row, and the
 * row replaced by the dequantized q * s. */
static void orc_quant_row(int n, double* a) {
  uint16_t* bits = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n);
  uint8_t* q = (uint8_t*)malloc((size_t)n);
  float* s = (float*)malloc(sizeof(float) * (size_t)(n / 128));
  if (!bits || !q || !s) abort();
  for (int i = 0; i < n; ++i) {
    float f = (float)a[i];
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u); /* round to nearest even on the upper half */
    bits[i] = (uint16_t)(u >> 16);
  }
  oracle_quant_act_e4m3(1, n, bits, q, s);
  for (int i = 0; i < n; ++i) a[i] = oracle_fp8_e4m3fn_to_f64(q[i]) * (double)s[i / 128];
  free(bits);
  free(q);
  free(s);
}

/* Finite float inputs only: the nearest E4M3FN codes of n fp32 values |v| <= 448
 * (the rounding step of Q alone, for the pins). */
int oracle_e4m3_round(const float* v, int64_t n, uint8_t* q) {
  double vals[127];
  for (int c = 0; c <= 126; ++c) vals[c] = oracle_fp8_e4m3fn_to_f64((uint8_t)c);
  for (int64_t i = 0; i < n; ++i) {
    if (!(fabsf(v[i]) <= 448.0f)) return -1;
    q[i] = orc_e4m3_nearest(v[i], vals);
  }
  return 0;
}

/* -------------------------------------------------------------- O1: route -- */

/* For each token: k passes over e = 0..E-1, each taking the largest logit not yet
 * chosen; a later expert replaces the current pick only when strictly greater, so
 * ties go to the lower index (and -0 ties +0).  Weights: renormalize != 0 gives
 * the softmax over the k chosen logits, w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0);
 * renormalize == 0 gives those experts' values of the softmax over all E logits. */
int oracle_route_topk(int B, int E, int k, int renormalize, const float* logits,
                      int32_t* ids, double* w) {
  if (B < 0 || E < 1 || k < 1 || k > E) return -1;
  char* used = (char*)malloc((size_t)E);
  if (!used) return -2;
  for (int t = 0; t < B; ++t) {
    const float* l = logits + (int64_t)t * E;
    memset(used, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (used[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      used[best] = 1;
      ids[(int64_t)t * k + j] = best;
    }
    double top = (double)l[ids[(int64_t)t * k]];
    double den = 0.0;
    if (renormalize) {
      for (int j = 0; j < k; ++j) den += exp((double)l[ids[(int64_t)t * k + j]] - top);
    } else {
      for (int e = 0; e < E; ++e) den += exp((double)l[e] - top);
    }
    for (int j = 0; j < k; ++j)
      w[(int64_t)t * k + j] = exp((double)l[ids[(int64_t)t * k + j]] - top) / den;
  }
  free(used);
  return 0;
}

/* ------------------------------------------------------------- O2: counts -- */

/* n_e for the local experts [e0, e0 + E_loc); slots routed elsewhere are ignored. */
void oracle_counts(int B, int k, int e0, int E_loc, const int32_t* ids, int32_t* counts) {
  for (int e = 0; e < E_loc; ++e) counts[e] = 0;
  for (int64_t s = 0; s < (int64_t)B * k; ++s) {
    int e = ids[s] - e0;
    if (e >= 0 && e < E_loc) counts[e] += 1;
  }
}

/* ------------------------------------------------------------- O3: select -- */

static int64_t orc_ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* For configuration v with b[v] token rows per tile, q1[v] / q2[v] tiles per
 * row-block in the gate/up and down phases and S1[v] / S2[v] tiles resident per
 * wave of the GPU:
 *   rt   = sum_e ceil(n_e / b)                 (row-blocks)
 *   T_p  = q_p * rt,  T = T_1 + T_2            (tiles, Eq. 1 summed over phases)
 *   W    = ceil(T_1 / S_1) + ceil(T_2 / S_2)   (waves, Eq. 1)
 *   A    = #{e : n_e > 0}                      (active experts)
 *   t_v  = fmaf(th3, A, fmaf(th2, T, fmaf(th1, W, th0)))   in fp32 (Eq. 3)
 * Returns argmin_v t_v, the first index on ties (Eq. 2); -1 on bad input.
 * feat[v*3 + 0..2] receives W, T, A and t_hat[v] the prediction. */
int oracle_select(int E_loc, const int32_t* counts, int V, const int32_t* b, const int32_t* q1,
                  const int32_t* q2, const int32_t* S1, const int32_t* S2, const float* theta,
                  float* t_hat, int32_t* feat) {
  int best = -1;
  float best_t = 0.0f;
  int64_t A = 0;
  for (int e = 0; e < E_loc; ++e) A += counts[e] > 0;
  for (int v = 0; v < V; ++v) {
    if (b[v] < 1 || S1[v] < 1 || S2[v] < 1) return -1;
    int64_t rt = 0;
    for (int e = 0; e < E_loc; ++e) rt += orc_ceil_div(counts[e], b[v]);
    int64_t T1 = (int64_t)q1[v] * rt, T2 = (int64_t)q2[v] * rt;
    int64_t T = T1 + T2;
    int64_t W = orc_ceil_div(T1, S1[v]) + orc_ceil_div(T2, S2[v]);
    if (T >= (1 << 24) || W >= (1 << 24) || A >= (1 << 24)) return -1; /* exact in fp32 */
    const float* th = theta + 4 * v;
    float t = fmaf(th[3], (float)A, fmaf(th[2], (float)T, fmaf(th[1], (float)W, th[0])));
    if (t_hat) t_hat[v] = t;
    if (feat) {
      feat[3 * v + 0] = (int32_t)W;
      feat[3 * v + 1] = (int32_t)T;
      feat[3 * v + 2] = (int32_t)A;
    }
    if (best < 0 || t < best_t) {
      best = v;
      best_t = t;
    }
  }
  return best;
}

/* -------------------------------------------------------------- O4: align -- */

/* Experts in ascending local index; inside one expert its slots s = t*k + j in
 * ascending order, then -1 up to the next multiple of b rows.  block_expert[i] is
 * the local expert of row-block i, slot_pos[s] the row of slot s (-1 when s is
 * routed to a non-local expert).  Returns the padded row count R, or -1 when R
 * would exceed cap. */
int64_t oracle_align(int B, int k, int e0, int E_loc, const int32_t* ids, int b,
                     int32_t* sorted_slots, int64_t cap, int32_t* block_expert,
                     int32_t* num_blocks, int32_t* slot_pos) {
  int64_t S = (int64_t)B * k, off = 0;
  for (int64_t s = 0; s < S; ++s) slot_pos[s] = -1;
  for (int e = 0; e < E_loc; ++e) {
    int64_t n = 0;
    for (int64_t s = 0; s < S; ++s) {
      if (ids[s] - e0 != e) continue;
      if (off + n >= cap) return -1;
      sorted_slots[off + n] = (int32_t)s;
      slot_pos[s] = (int32_t)(off + n);
      ++n;
    }
    int64_t padded = orc_ceil_div(n, b) * b;
    if (off + padded > cap) return -1;
    for (int64_t i = n; i < padded; ++i) sorted_slots[off + i] = -1;
    for (int64_t blk = 0; blk < padded / b; ++blk) block_expert[off / b + blk] = e;
    off += padded;
  }
  *num_blocks = (int32_t)(off / b);
  return off;
}

/* ---------------------------------------------------------------- O5: ffn -- */

/* Expert e's output for one token row x (length H), in fp64:
 *   g_i = sum_h x_h W1[e][i][h],  u_i = sum_h x_h W3[e][i][h]
 *   a_i = g_i / (1 + exp(-g_i)) * u_i
 *   y_d = sum_i a_i W2[e][d][i]                                               */
static void orc_expert_ffn(int H, int I, const double* x, const void* w1, const void* w3,
                           const void* w2, int wdt, const float* s1, const float* s3,
                           const float* s2, int e, double* a, double* y, int hq) {
  for (int i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    for (int h = 0; h < H; ++h) {
      g += x[h] * orc_weight(w1, wdt, s1, e, I, H, i, h);
      u += x[h] * orc_weight(w3, wdt, s3, e, I, H, i, h);
    }
    a[i] = g / (1.0 + exp(-g)) * u;
  }
  if (hq) orc_quant_row(I, a);
  for (int d = 0; d < H; ++d) {
    double acc = 0.0;
    for (int i = 0; i < I; ++i) acc += a[i] * orc_weight(w2, wdt, s2, e, H, I, d, i);
    y[d] = acc;
  }
}

/* y[n][H] for n (token, local expert) pairs. */
int oracle_ffn_slots(int H, int I, const void* x, int xdt, const void* w1, const void* w3,
                     const void* w2, int wdt, const float* s1, const float* s3, const float* s2,
                     int n, const int32_t* tok, const int32_t* exp_local, double* y,
                     int nthreads, int hq) {
  int err = 0;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1) reduction(| : err)
  for (int i = 0; i < n; ++i) {
    double* xr = (double*)malloc(sizeof(double) * (size_t)H);
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    if (!xr || !a) {
      err |= 1;
    } else {
      for (int h = 0; h < H; ++h) xr[h] = orc_act(x, xdt, (int64_t)tok[i] * H + h);
      orc_expert_ffn(H, I, xr, w1, w3, w2, wdt, s1, s3, s2, exp_local[i], a, y + (int64_t)i * H, hq);
    }
    free(xr);
    free(a);
  }
  return err ? -2 : 0;
}

/* ------------------------------------------------------------ O6: combine -- */

/* Whole layer for a list of tokens (all of them, or a sample): for each listed
 * token t, y_t = sum over j = 0..k-1 with ids[t][j] local of w[t][j] * FFN_e(x_t),
 * accumulated in j order; tokens with no local expert give 0.  ids/w are O1's. */
int oracle_layer_tokens(int H, int I, int k, int e0, int E_loc, const void* x, int xdt,
                        const void* w1, const void* w3, const void* w2, int wdt, const float* s1,
                        const float* s3, const float* s2, const int32_t* ids, const double* w,
                        int n_tok, const int32_t* tokens, double* Y, int nthreads, int hq,
                        int n_shared) {
  int err = 0;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1) reduction(| : err)
  for (int i = 0; i < n_tok; ++i) {
    int t = tokens[i];
    double* xr = (double*)malloc(sizeof(double) * (size_t)H);
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    double* ys = (double*)malloc(sizeof(double) * (size_t)H);
    double* out = Y + (int64_t)i * H;
    if (!xr || !a || !ys) {
      err |= 1;
    } else {
      for (int h = 0; h < H; ++h) xr[h] = orc_act(x, xdt, (int64_t)t * H + h);
      for (int d = 0; d < H; ++d) out[d] = 0.0;
      for (int j = 0; j < k; ++j) {
        int e = ids[(int64_t)t * k + j] - e0;
        if (e < 0 || e >= E_loc) continue;
        orc_expert_ffn(H, I, xr, w1, w3, w2, wdt, s1, s3, s2, e, a, ys, hq);
        double g = w[(int64_t)t * k + j];
        for (int d = 0; d < H; ++d) out[d] += g * ys[d];
      }
      for (int i = 0; i < n_shared; ++i) {  /* the shared lanes, weight 1 */
        orc_expert_ffn(H, I, xr, w1, w3, w2, wdt, s1, s3, s2, E_loc + i, a, ys, hq);
        for (int d = 0; d < H; ++d) out[d] += ys[d];
      }
    }
    free(xr);
    free(a);
    free(ys);
  }
  return err ? -2 : 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
