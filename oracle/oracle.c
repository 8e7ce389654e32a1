/*
 * CPU oracle for the routed-expert FFN at decode time.  TEST INFRASTRUCTURE:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  It shares no source, header, table or helper with the HIP
 * library; it is plain scalar C99 with every floating-point result accumulated
 * in fp64.
 *
 * What is computed (the "MUL_MAT_ID" of page "Kimi-K3 on 2x A40 -- measured
 * findings", section "Why the placement experiments all looked the same": each
 * token multiplies by the matrices of the experts it selected), with the layer
 * structure of page "SparkInfer-K3", section "How the TP module works" (one
 * router over replicated weights picks the top-16 experts, the selected experts
 * are evaluated, and their outputs are summed) and page "Kimi-K3 on the same
 * pod, two engines", sections "Same hardware, same weights" and "Reason 1"
 * (routing and the final add sit beside the expert work; partial sums are added
 * in a fixed order):
 *
 *   logits  L[t][e] = sum_h x[t][h] * W_r[e][h]                    (fp64)
 *   select  S_t = the k experts with the largest L[t][e], ties to the lower
 *           index, listed by (L desc, index asc)
 *   weights w_s = sigmoid(L[t][S_t[s]]) / sum_r sigmoid(L[t][S_t[r]])
 *   expert  g = Wg x, u = Wu x, h = silu(g) * u, y = Wd h        (fp64)
 *   combine out[t] = sum_{s=0}^{k-1} w_s * y_s                     (fp64)
 *
 * The pages only name the weight formats (MXFP4 for the 3584->3072 expert
 * shapes of the microbenchmark, NVFP4 for the K3 checkpoint).  Their element
 * encodings are the public OCP ones: e2m1 codes, e8m0 and fp8-e4m3 scales.
 * The sigmoid-renormalised routing and SwiGLU are the plainest readings the
 * workloads state; the pages name no routing function.
 *
 * Nothing here is blocked, fused or reordered: each sum runs over its index in
 * increasing order.  OpenMP only splits independent output rows over threads,
 * so every result is the same for any thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

/* ---------------------------------------------------------------------------
 * O1  Element encodings (OCP Microscaling v1.0 / OCP 8-bit floating point).
 * ------------------------------------------------------------------------- */

/* e2m1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN.
 * exponent field 0 is subnormal: 0.5 * m. */
EXPORT double orc_e2m1(int code) {
  const int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* e8m0: an unsigned power-of-two exponent with bias 127; 0xFF is NaN. */
EXPORT double orc_e8m0(int byte) {
  byte &= 0xFF;
  if (byte == 0xFF) return NAN;
  return ldexp(1.0, byte - 127);
}

/* fp8 e4m3 ("FN"): sign, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; exponent field 0 is subnormal (m/8)*2^-6. */
EXPORT double orc_e4m3(int byte) {
  byte &= 0xFF;
  const int s = byte >> 7, E = (byte >> 3) & 15, m = byte & 7;
  double mag;
  if (E == 15 && m == 7) return NAN;
  if (E == 0) mag = ldexp(m / 8.0, -6);
  else mag = ldexp(1.0 + m / 8.0, E - 7);
  return s ? -mag : mag;
}

/* Element j of a packed row: two codes per byte, element 2i in bits 3..0 and
 * element 2i+1 in bits 7..4. */
static int code_at(const uint8_t *row, int64_t j) {
  const uint8_t b = row[j >> 1];
  return (j & 1) ? (b >> 4) : (b & 15);
}

/* fp64 -> fp32 with one IEEE-754 round-to-nearest-even (C Annex F conversion:
 * values beyond the fp32 range become +-inf, NaN stays NaN). */
static float round_f32(double v) { return (float)v; }

/* ---------------------------------------------------------------------------
 * O2  Dequantisation to fp32: the exact real product, rounded once.
 * ------------------------------------------------------------------------- */

/* MX: w[n][j] = e2m1(code) * 2^(b-127), one e8m0 byte b per 32 elements of a
 * row.  The product is exact in fp64. */
EXPORT void orc_dequant_mx(const uint8_t *codes, const uint8_t *scales, int64_t N,
                           int64_t K, float *out) {
  for (int64_t n = 0; n < N; ++n) {
    const uint8_t *crow = codes + n * (K / 2);
    const uint8_t *srow = scales + n * (K / 32);
    for (int64_t j = 0; j < K; ++j)
      out[n * K + j] = round_f32(orc_e2m1(code_at(crow, j)) * orc_e8m0(srow[j / 32]));
  }
}

/* NV: w[n][j] = e2m1(code) * e4m3(s) * g, one e4m3 byte s per 16 elements and
 * one fp32 g per tensor.  e2m1*e4m3 has at most 6 significant bits and g 24,
 * so the product is exact in fp64 and is rounded once. */
EXPORT void orc_dequant_nv(const uint8_t *codes, const uint8_t *scales, float g,
                           int64_t N, int64_t K, float *out) {
  for (int64_t n = 0; n < N; ++n) {
    const uint8_t *crow = codes + n * (K / 2);
    const uint8_t *srow = scales + n * (K / 16);
    for (int64_t j = 0; j < K; ++j)
      out[n * K + j] =
          round_f32(orc_e2m1(code_at(crow, j)) * orc_e4m3(srow[j / 16]) * (double)g);
  }
}

/* ---------------------------------------------------------------------------
 * O3  Router logits.
 * ------------------------------------------------------------------------- */
EXPORT void orc_router(const float *x, const float *Wr, int C, int H, int E,
                       double *logits) {
  for (int t = 0; t < C; ++t) {
    #pragma omp parallel for schedule(static)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h) acc += (double)x[(int64_t)t * H + h] * (double)Wr[(int64_t)e * H + h];
      logits[(int64_t)t * E + e] = acc;
    }
  }
}

/* ---------------------------------------------------------------------------
 * O4  Selection: k passes, each taking the best remaining expert under the
 * order (value desc, index asc).  NaN ranks below every number; -0 == +0.
 * ------------------------------------------------------------------------- */
static int better(double a, int ia, double b, int ib) {
  const int na = isnan(a), nb = isnan(b);
  if (na || nb) {
    if (na && nb) return ia < ib;
    return nb;            /* a number beats NaN */
  }
  if (a > b) return 1;
  if (a < b) return 0;
  return ia < ib;        /* equal values (including -0 vs +0): lower index */
}

EXPORT void orc_topk(const double *v, int E, int k, int32_t *idx) {
  char *taken = (char *)calloc((size_t)E, 1);
  for (int s = 0; s < k; ++s) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || better(v[e], e, v[best], best)) best = e;
    }
    taken[best] = 1;
    idx[s] = best;
  }
  free(taken);
}

/* The same selection on fp32 values (used where both sides must decide on
 * identical fp32 logits). */
EXPORT void orc_topk_f32(const float *v, int E, int k, int32_t *idx) {
  double *d = (double *)malloc(sizeof(double) * (size_t)E);
  for (int e = 0; e < E; ++e) d[e] = (double)v[e];  /* exact widening */
  orc_topk(d, E, k, idx);
  free(d);
}

/* ---------------------------------------------------------------------------
 * O5  Routing weights: sigmoid scores renormalised over the selected set.
 * ------------------------------------------------------------------------- */
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

EXPORT void orc_route_weights(const double *l_sel, int k, double *w) {
  double sum = 0.0;
  for (int s = 0; s < k; ++s) sum += sigmoid(l_sel[s]);
  for (int s = 0; s < k; ++s) w[s] = sigmoid(l_sel[s]) / sum;
}

/* ---------------------------------------------------------------------------
 * O6  One expert's SwiGLU FFN on one token, weights as their fp32 values.
 *     Wg, Wu: [I][H]; Wd: [H][I]; x: [H]; y: [H].
 * ------------------------------------------------------------------------- */
EXPORT double orc_silu(double z) { return z * sigmoid(z); }

EXPORT void orc_expert_ffn(const float *Wg, const float *Wu, const float *Wd,
                           const float *x, int H, int I, double *y) {
  double *hbuf = (double *)malloc(sizeof(double) * (size_t)I);
  #pragma omp parallel for schedule(static)
  for (int j = 0; j < I; ++j) {
    double g = 0.0, u = 0.0;
    for (int h = 0; h < H; ++h) {
      g += (double)Wg[(int64_t)j * H + h] * (double)x[h];
      u += (double)Wu[(int64_t)j * H + h] * (double)x[h];
    }
    hbuf[j] = orc_silu(g) * u;
  }
  #pragma omp parallel for schedule(static)
  for (int o = 0; o < H; ++o) {
    double acc = 0.0;
    for (int j = 0; j < I; ++j) acc += (double)Wd[(int64_t)o * I + j] * hbuf[j];
    y[o] = acc;
  }
  free(hbuf);
}

/* The intermediate activation alone (h = silu(Wg x) * (Wu x)), for tests of
 * the first half of the expert. */
EXPORT void orc_expert_hidden(const float *Wg, const float *Wu, const float *x, int H,
                              int I, double *h) {
  #pragma omp parallel for schedule(static)
  for (int j = 0; j < I; ++j) {
    double g = 0.0, u = 0.0;
    for (int k = 0; k < H; ++k) {
      g += (double)Wg[(int64_t)j * H + k] * (double)x[k];
      u += (double)Wu[(int64_t)j * H + k] * (double)x[k];
    }
    h[j] = orc_silu(g) * u;
  }
}

/* ---------------------------------------------------------------------------
 * O7  Weighted combine in slot order: out[o] = sum_s w[s] * y[s][o].
 *     y: [k][H] fp64.
 * ------------------------------------------------------------------------- */
EXPORT void orc_combine(const double *w, const double *y, int k, int H, double *out) {
  for (int o = 0; o < H; ++o) {
    double acc = 0.0;
    for (int s = 0; s < k; ++s) acc += w[s] * y[(int64_t)s * H + o];
    out[o] = acc;
  }
}

/* Threads OpenMP would use (1 when built without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
EXPORT int orc_threads(void) { return omp_get_max_threads(); }
EXPORT void orc_set_threads(int n) { omp_set_num_threads(n); }
#else
EXPORT int orc_threads(void) { return 1; }
EXPORT void orc_set_threads(int n) { (void)n; }
#endif
