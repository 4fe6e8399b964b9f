/*
 * CPU oracle for one MoE-layer forward pass.  TEST INFRASTRUCTURE ONLY:
 * it is used by tests/, by __graft_entry__.smoke() and by bench.py's
 * cpu_baseline leg, never by the product path.  It shares no code with the
 * HIP library.
 *
 * It is the plain definition, written slowly and in double precision:
 *
 *  - router: logits[t][e] = fp32( sum_i x[t][i] * Wg[i][e]  (+ b[e]) )
 *    (a router maps every token to its experts: HARMOEny article,
 *    yejing.asia, section 3.3 step one; the gating network runs on the GPU:
 *    GPU-cache article, coreui.cn, section 3.1).
 *  - top-k: experts ranked by (logit descending, expert index ascending),
 *    NaN below every number, +0 == -0; the k first are taken, slot 0 first.
 *  - gate weights: softmax over the k selected logits,
 *    w_j = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), in double, stored fp32.
 *    (Equal in exact arithmetic to a softmax over all E renormalised over the
 *    selected k.)
 *  - dispatch: counts, exclusive offsets and the stable counting-sort
 *    permutation of assignment ids a = t*k + j by expert (HARMOEny article,
 *    section 3.3 step four: tokens are sent to their experts).
 *  - expert: the two-layer MLP x*W1*W2 with W1 m x p and W2 p x m (HARMOEny
 *    article, section 3.2 "expert prefetch"), with ReLU between the two
 *    matrices, or its SwiGLU form h = SiLU(x*W1) * (x*W3), o = h*W2.  int8
 *    weights stand for q[i][n] * s[n] (per output channel n), fp8 weights
 *    for e4m3(code) * s[n], MXFP4 weights for e2m1(code) times the E8M0
 *    scale of their block of 32 consecutive i (see weight() below).  With
 *    fp8 activations (ORC_FP8A8) each token's row is first quantised to
 *    E4M3 with one power-of-two scale per row (quant_row_e4m3 below), with
 *    int8 activations (ORC_I8A8) to int8 likewise (quant_row_i8); the router
 *    still reads the row unquantised.  Every dot
 *    product of length n is a0*b0 followed by n-1 multiply-adds, and an
 *    operation counter records each multiply and each add.
 *  - combine: y[t] = sum over the token's selections, in ascending expert
 *    index, of w * o  (HARMOEny article, section 3.3 step six: finished
 *    tokens are collected).
 *
 *  - neighbouring ops (DeepSpeed-Inference summary, datalearner.com, section
 *    4: the post-attention layer norm fused with the intermediate GeMM, and
 *    the bias and residual addition; section 2: a layer norm's reductions
 *    run along the row inside one tile).  Layer norm of a row x of m:
 *    mu = sum x / m, var = sum (x - mu)^2 / m, out = (x - mu) / sqrt(var +
 *    eps) * gamma + beta; the RMS form drops the mean and beta:
 *    out = x / sqrt(sum x^2 / m + eps) * gamma.  The residual is added to
 *    the combined output (in the tests, beside the layer).
 *
 * Return codes: 0 on success, -1 on a bad argument.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element access ----------------------------------------------------- */

static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Activation element i of a fp32 or bf16 array. */
static double act_at(const void* x, int dtype, int64_t i) {
  if (dtype == ORC_F32) return (double)((const float*)x)[i];
  return bf16_bits_to_double(((const uint16_t*)x)[i]);
}

/* The 8-bit float E4M3 of the OCP 8-bit floating point format (OFP8,
 * "E4M3FN"): sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
 * field 0 holds the subnormals m * 2^-9; no infinities; S.1111.111 is NaN, so
 * the largest finite magnitude is 1.75 * 2^8 = 448. */
static double e4m3_value(uint8_t c) {
  const int sign = c >> 7, ex = (c >> 3) & 15, mt = c & 7;
  if (ex == 15 && mt == 7) return NAN;
  const double v = ex == 0 ? mt * ldexp(1.0, -9) : (1.0 + mt / 8.0) * ldexp(1.0, ex - 7);
  return sign ? -v : v;
}

/* The 4-bit float E2M1 of the OCP microscaling (MX) formats: sign bit, 2
 * exponent bits with bias 1, 1 mantissa bit; exponent field 0 holds the
 * subnormal 0.5 m; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Codes are the low
 * nibble of a byte (bit 3 the sign). */
static double e2m1_value(uint8_t c) {
  const int sign = (c >> 3) & 1, ex = (c >> 1) & 3, mt = c & 1;
  const double v = ex == 0 ? 0.5 * mt : (1.0 + 0.5 * mt) * ldexp(1.0, ex - 1);
  return sign ? -v : v;
}

/* The shared scale E8M0 of the MX formats: 2^(E - 127); E = 255 is NaN. */
static double e8m0_value(uint8_t E) { return E == 255 ? NAN : ldexp(1.0, (int)E - 127); }

/* E4M3 code of a finite v: round to nearest, ties to even, on the format's
 * grid (quantum 2^-9 below the smallest normal 2^-6, 2^(e-3) in [2^e,
 * 2^(e+1))), magnitudes that would round above 448 (the largest finite
 * value; 480 does not exist) saturating to 448.  Negative zero keeps its
 * sign. */
static uint8_t e4m3_encode(double v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0;
  const double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) {
    const double q = nearbyint(a * 512.0); /* multiples of 2^-9; 8 is the smallest normal */
    return sign | (uint8_t)q;
  }
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): a in [2^(e-1), 2^e) */
  e -= 1;
  double q = nearbyint(ldexp(a, 3 - e)); /* in [8, 16] */
  if (q == 16.0) {
    q = 8.0;
    e += 1;
  }
  if (e > 8 || (e == 8 && q > 14.0)) return sign | 0x7E;
  return sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8));
}

/* The smallest X with amax <= qmax * 2^X (amax > 0). */
static int pow2_exponent(double amax, double qmax) {
  int X = (int)ceil(log2(amax / qmax));
  while (amax > qmax * ldexp(1.0, X)) ++X; /* guard the boundary against log2's rounding */
  while (amax <= qmax * ldexp(1.0, X - 1)) --X;
  return X;
}

/* One row of m activations quantised to E4M3 with a per-row power-of-two
 * scale: s = 2^X with X the smallest integer such that max|x| <= 448 * 2^X
 * (so no element saturates), code = e4m3(x / s) (the division by a power of
 * two is exact), and the value the experts read is e4m3(code) * s, which
 * bf16 holds exactly.  A row of zeros quantises to zeros (s = 1). */
static void quant_row_e4m3(const double* x, int m, double* out, uint8_t* codes, float* scale) {
  double amax = 0.0;
  for (int i = 0; i < m; ++i) amax = fabs(x[i]) > amax ? fabs(x[i]) : amax;
  const int X = amax > 0.0 ? pow2_exponent(amax, 448.0) : 0;
  const double sc = ldexp(1.0, X);
  for (int i = 0; i < m; ++i) {
    const uint8_t c = e4m3_encode(x[i] / sc);
    if (codes) codes[i] = c;
    out[i] = e4m3_value(c) * sc;
  }
  if (scale) *scale = (float)sc;
}

/* One row quantised to int8 with a per-row power-of-two scale s = 2^X, X the
 * smallest integer with max|x| <= 127 * 2^X: q = x / s rounded to the nearest
 * integer, ties to even (|q| <= 127; the division is exact), value q * s
 * (exact in bf16: seven significant bits).  A row of zeros gives zeros
 * (s = 1). */
static void quant_row_i8(const double* x, int m, double* out, int8_t* codes, float* scale) {
  double amax = 0.0;
  for (int i = 0; i < m; ++i) amax = fabs(x[i]) > amax ? fabs(x[i]) : amax;
  const int X = amax > 0.0 ? pow2_exponent(amax, 127.0) : 0;
  const double sc = ldexp(1.0, X);
  for (int i = 0; i < m; ++i) {
    const double q = nearbyint(x[i] / sc);
    if (codes) codes[i] = (int8_t)q;
    out[i] = q * sc;
  }
  if (scale) *scale = (float)sc;
}

/* Weight (e, k, n) of a projection stored [E][K][N] (k along the reduction):
 *  - fp32, bf16: the stored value;
 *  - int8 (int4 as well: q in [-7, 7], one per byte): q * s[e][n], one fp32
 *    scale per output channel;
 *  - fp8: e4m3(code) * s[e][n], one fp32 scale per output channel;
 *  - MXFP4: e2m1(code) * e8m0(X[e][k / 32][n]): one E8M0 scale shared by the
 *    32 consecutive k of a column (the MX block of 32 elements). */
static double weight(const void* w, const void* s, int dtype, int64_t e, int64_t K, int64_t N, int64_t k,
                     int64_t n) {
  const int64_t i = (e * K + k) * N + n;
  switch (dtype) {
    case ORC_F32: return (double)((const float*)w)[i];
    case ORC_BF16: return bf16_bits_to_double(((const uint16_t*)w)[i]);
    case ORC_I8:
    case ORC_I8A8: return (double)((const int8_t*)w)[i] * (double)((const float*)s)[e * N + n];
    case ORC_FP8:
    case ORC_FP8A8: return e4m3_value(((const uint8_t*)w)[i]) * (double)((const float*)s)[e * N + n];
    default: return e2m1_value(((const uint8_t*)w)[i]) * e8m0_value(((const uint8_t*)s)[(e * (K / 32) + k / 32) * N + n]);
  }
}

int orc_weight_value(const void* w, const void* s, int dtype, int64_t e, int64_t K, int64_t N, int64_t k, int64_t n,
                     double* out) {
  if (!w || !out || dtype < ORC_F32 || dtype > ORC_I8A8) return -1;
  if (dtype >= ORC_I8 && !s) return -1;
  if (dtype == ORC_MXFP4 && K % 32) return -1;
  *out = weight(w, s, dtype, e, K, N, k, n);
  return 0;
}

int orc_e4m3_encode(const float* v, int64_t n, uint8_t* codes) {
  if ((!v || !codes) && n > 0) return -1;
  for (int64_t i = 0; i < n; ++i) codes[i] = e4m3_encode((double)v[i]);
  return 0;
}

int orc_quant_rows_e4m3(const void* x, int x_dtype, int T, int m, double* out, uint8_t* codes, float* scales) {
  if (!x || !out || T < 0 || m < 1 || (x_dtype != ORC_F32 && x_dtype != ORC_BF16)) return -1;
  double* xr = (double*)malloc(sizeof(double) * (size_t)m);
  if (!xr) return -1;
  for (int t = 0; t < T; ++t) {
    for (int c = 0; c < m; ++c) xr[c] = act_at(x, x_dtype, (int64_t)t * m + c);
    quant_row_e4m3(xr, m, out + (int64_t)t * m, codes ? codes + (int64_t)t * m : NULL, scales ? scales + t : NULL);
  }
  free(xr);
  return 0;
}

int orc_quant_rows_i8(const void* x, int x_dtype, int T, int m, double* out, int8_t* codes, float* scales) {
  if (!x || !out || T < 0 || m < 1 || (x_dtype != ORC_F32 && x_dtype != ORC_BF16)) return -1;
  double* xr = (double*)malloc(sizeof(double) * (size_t)m);
  if (!xr) return -1;
  for (int t = 0; t < T; ++t) {
    for (int c = 0; c < m; ++c) xr[c] = act_at(x, x_dtype, (int64_t)t * m + c);
    quant_row_i8(xr, m, out + (int64_t)t * m, codes ? codes + (int64_t)t * m : NULL, scales ? scales + t : NULL);
  }
  free(xr);
  return 0;
}

/* ---- router ------------------------------------------------------------- */

int orc_router_logits(const void* x, int x_dtype, const float* wg, const float* bias, int T, int m, int E,
                      float* logits) {
  if (T < 0 || m < 1 || E < 1 || (T > 0 && (!x || !wg || !logits))) return -1;
  if (x_dtype != ORC_F32 && x_dtype != ORC_BF16) return -1;
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      double s = act_at(x, x_dtype, (int64_t)t * m) * (double)wg[e];
      for (int i = 1; i < m; ++i) s += act_at(x, x_dtype, (int64_t)t * m + i) * (double)wg[(int64_t)i * E + e];
      if (bias) s += (double)bias[e];
      logits[(int64_t)t * E + e] = (float)s;
    }
  }
  return 0;
}

/* ---- norm of the layer's input rows ------------------------------------- */

int orc_norm(const void* x, int x_dtype, int T, int m, int kind, const float* gamma, const float* beta, double eps,
             double* out) {
  if (T < 0 || m < 1 || (T > 0 && (!x || !gamma || !out)) || eps < 0) return -1;
  if (x_dtype != ORC_F32 && x_dtype != ORC_BF16) return -1;
  if (kind != ORC_NORM_LAYER && kind != ORC_NORM_RMS) return -1;
  for (int t = 0; t < T; ++t) {
    const int64_t r = (int64_t)t * m;
    double mu = 0.0;
    if (kind == ORC_NORM_LAYER) {
      for (int i = 0; i < m; ++i) mu += act_at(x, x_dtype, r + i);
      mu /= m;
    }
    double ss = 0.0;
    for (int i = 0; i < m; ++i) {
      const double d = act_at(x, x_dtype, r + i) - mu;
      ss += d * d;
    }
    const double den = sqrt(ss / m + eps);
    for (int i = 0; i < m; ++i) {
      double v = (act_at(x, x_dtype, r + i) - mu) / den * (double)gamma[i];
      if (kind == ORC_NORM_LAYER && beta) v += (double)beta[i];
      out[r + i] = v;
    }
  }
  return 0;
}

/* ---- top-k and gate weights --------------------------------------------- */

/* 1 if expert a (logit va) ranks before expert b (logit vb). */
static int ranks_before(float va, int a, float vb, int b) {
  const int na = isnan(va), nb = isnan(vb);
  if (na || nb) {
    if (na && nb) return a < b;
    return nb; /* a number ranks before NaN */
  }
  if (va > vb) return 1;
  if (va < vb) return 0;
  return a < b; /* equal values (including +0 and -0): lower index first */
}

int orc_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w) {
  if (T < 0 || E < 1 || E > ORC_MAX_E || k < 1 || k > E) return -1;
  int order[ORC_MAX_E];
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (int64_t)t * E;
    /* stable insertion sort of 0..E-1 by the ranking */
    for (int e = 0; e < E; ++e) {
      int j = e;
      while (j > 0 && ranks_before(l[e], e, l[order[j - 1]], order[j - 1])) {
        order[j] = order[j - 1];
        --j;
      }
      order[j] = e;
    }
    const double l0 = (double)l[order[0]];
    double denom = 0.0;
    for (int j = 0; j < k; ++j) denom += exp((double)l[order[j]] - l0);
    for (int j = 0; j < k; ++j) {
      idx[(int64_t)t * k + j] = order[j];
      w[(int64_t)t * k + j] = (float)(exp((double)l[order[j]] - l0) / denom);
    }
  }
  return 0;
}

/* ---- dispatch ----------------------------------------------------------- */

int orc_dispatch(const int32_t* idx, int T, int E, int k, int32_t* counts, int32_t* offsets, int32_t* perm,
                 int32_t* inv_perm) {
  if (T < 0 || E < 1 || k < 1) return -1;
  const int64_t n = (int64_t)T * k;
  for (int64_t a = 0; a < n; ++a)
    if (idx[a] < 0 || idx[a] >= E) return -1;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t a = 0; a < n; ++a) counts[idx[a]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* cursor = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  if (!cursor) return -1;
  for (int64_t a = 0; a < n; ++a) {
    const int e = idx[a];
    perm[offsets[e] + cursor[e]] = (int32_t)a;
    cursor[e] += 1;
  }
  free(cursor);
  for (int64_t r = 0; r < n; ++r) inv_perm[perm[r]] = (int32_t)r;
  return 0;
}

/* ---- one expert on one activation row ----------------------------------- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* x[m] (double) -> o[m] (double) through expert e.  Scratch: g[p], u[p].
 * ops[0] += multiplies+adds of the dot products, ops[1] += activation
 * evaluations (ReLU or SiLU), ops[2] += the SwiGLU elementwise products. */
static void expert_row(const orc_experts* X, int e, const double* x_in, double* g, double* u, double* o,
                       double* xq, uint64_t ops[3]) {
  const int m = X->m, p = X->p;
  const int swiglu = (X->kind == ORC_SWIGLU);
  const int dt = X->w_dtype;
  /* fp8 activations: the first projection reads the row quantised per token */
  const double* x = x_in;
  if (dt == ORC_FP8A8 || dt == ORC_I8A8) {
    if (dt == ORC_FP8A8)
      quant_row_e4m3(x_in, m, xq, NULL, NULL);
    else
      quant_row_i8(x_in, m, xq, NULL, NULL);
    x = xq;
  }

  /* g = x*W1 (and u = x*W3): every g[n] is the length-m dot product in
   * increasing i, started with the i = 0 product.  The counters tick once
   * per multiply and once per add actually performed. */
  uint64_t mul = 0, add = 0, act = 0, prod = 0;
  for (int n = 0; n < p; ++n) {
    g[n] = x[0] * weight(X->w1, X->s1, dt, e, m, p, 0, n);
    mul += 1;
    if (swiglu) {
      u[n] = x[0] * weight(X->w3, X->s3, dt, e, m, p, 0, n);
      mul += 1;
    }
  }
  for (int i = 1; i < m; ++i) {
    for (int n = 0; n < p; ++n) {
      g[n] += x[i] * weight(X->w1, X->s1, dt, e, m, p, i, n);
      mul += 1;
      add += 1;
      if (swiglu) {
        u[n] += x[i] * weight(X->w3, X->s3, dt, e, m, p, i, n);
        mul += 1;
        add += 1;
      }
    }
  }

  /* h overwrites g, kept in double (not rounded) */
  for (int n = 0; n < p; ++n) {
    if (swiglu) {
      g[n] = silu(g[n]) * u[n];
      prod += 1;
    } else {
      g[n] = g[n] > 0.0 ? g[n] : 0.0;
    }
    act += 1;
  }

  /* o = h*W2 */
  for (int j = 0; j < m; ++j) {
    o[j] = g[0] * weight(X->w2, X->s2, dt, e, p, m, 0, j);
    mul += 1;
  }
  for (int n = 1; n < p; ++n) {
    for (int j = 0; j < m; ++j) {
      o[j] += g[n] * weight(X->w2, X->s2, dt, e, p, m, n, j);
      mul += 1;
      add += 1;
    }
  }
  ops[0] += mul + add;
  ops[1] += act;
  ops[2] += prod;
}

static int check_experts(const orc_experts* X) {
  if (!X || X->m < 1 || X->p < 1 || X->E < 1 || !X->w1 || !X->w2) return -1;
  if (X->kind != ORC_RELU && X->kind != ORC_SWIGLU) return -1;
  if (X->kind == ORC_SWIGLU && !X->w3) return -1;
  if (X->w_dtype < ORC_F32 || X->w_dtype > ORC_I8A8) return -1;
  if (X->w_dtype >= ORC_I8 && (!X->s1 || !X->s2 || (X->kind == ORC_SWIGLU && !X->s3))) return -1;
  if (X->w_dtype == ORC_MXFP4 && (X->m % 32 || X->p % 32)) return -1;
  return 0;
}

int orc_expert_apply(const orc_experts* X, int e, const double* x, double* o, uint64_t* ops3) {
  if (check_experts(X) || e < 0 || e >= X->E) return -1;
  double* g = (double*)malloc(sizeof(double) * (size_t)X->p);
  double* u = (double*)malloc(sizeof(double) * (size_t)X->p);
  double* xq = (double*)malloc(sizeof(double) * (size_t)X->m);
  if (!g || !u || !xq) { free(g); free(u); free(xq); return -1; }
  uint64_t ops[3] = {0, 0, 0};
  expert_row(X, e, x, g, u, o, xq, ops);
  if (ops3) { ops3[0] += ops[0]; ops3[1] += ops[1]; ops3[2] += ops[2]; }
  free(g);
  free(u);
  free(xq);
  return 0;
}

/* Permuted expert rows: out[i] = FFN_{e}(x[perm[r]/k]) for r = rows[i], with
 * e the expert whose offsets segment holds r.  rows == NULL means all
 * T*k rows in order. */
int orc_expert_rows(const orc_experts* X, const void* x, int x_dtype, int T, int k, const int32_t* perm,
                    const int32_t* offsets, const int32_t* rows, int nrows, double* out, uint64_t* ops3) {
  if (check_experts(X) || T < 0 || k < 1 || (x_dtype != ORC_F32 && x_dtype != ORC_BF16)) return -1;
  const int m = X->m, p = X->p, E = X->E;
  const int64_t n_all = (int64_t)T * k;
  if (!rows) nrows = (int)n_all;
  int bad = 0;
  uint64_t o0 = 0, o1 = 0, o2 = 0;
#pragma omp parallel reduction(+ : o0, o1, o2) reduction(| : bad)
  {
    double* g = (double*)malloc(sizeof(double) * (size_t)p);
    double* u = (double*)malloc(sizeof(double) * (size_t)p);
    double* xr = (double*)malloc(sizeof(double) * (size_t)m);
    double* xq = (double*)malloc(sizeof(double) * (size_t)m);
    if (!g || !u || !xr || !xq) bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < nrows; ++i) {
      if (bad) continue;
      const int64_t r = rows ? rows[i] : i;
      if (r < 0 || r >= n_all) { bad = 1; continue; }
      int e = 0;
      while (e < E && !(offsets[e] <= r && r < offsets[e + 1])) ++e;
      if (e == E) { bad = 1; continue; }
      const int64_t t = perm[r] / k;
      for (int c = 0; c < m; ++c) xr[c] = act_at(x, x_dtype, t * m + c);
      uint64_t ops[3] = {0, 0, 0};
      expert_row(X, e, xr, g, u, out + (int64_t)i * m, xq, ops);
      o0 += ops[0]; o1 += ops[1]; o2 += ops[2];
    }
    free(g); free(u); free(xr); free(xq);
  }
  if (ops3) { ops3[0] += o0; ops3[1] += o1; ops3[2] += o2; }
  return bad ? -1 : 0;
}

/* ---- combine ------------------------------------------------------------ */

/* Selections of token t in ascending expert index (ties keep slot order). */
static void ascending_slots(const int32_t* idx_t, int k, int* slot) {
  for (int j = 0; j < k; ++j) {
    int i = j;
    while (i > 0 && idx_t[slot[i - 1]] > idx_t[j]) { slot[i] = slot[i - 1]; --i; }
    slot[i] = j;
  }
}

int orc_combine(const double* y_perm, const int32_t* inv_perm, const int32_t* idx, const float* w, int T, int m,
                int k, double* y) {
  if (T < 0 || m < 1 || k < 1 || k > ORC_MAX_E) return -1;
  int slot[ORC_MAX_E];
  for (int t = 0; t < T; ++t) {
    ascending_slots(idx + (int64_t)t * k, k, slot);
    double* yt = y + (int64_t)t * m;
    for (int c = 0; c < m; ++c) yt[c] = 0.0;
    for (int s = 0; s < k; ++s) {
      const int j = slot[s];
      const double wj = (double)w[(int64_t)t * k + j];
      const double* o = y_perm + (int64_t)inv_perm[(int64_t)t * k + j] * m;
      for (int c = 0; c < m; ++c) yt[c] += wj * o[c];
    }
  }
  return 0;
}

/* ---- end to end on selected tokens -------------------------------------- */

/*
 * y[i] for token tokens[i], straight from the definition: its logits (or the
 * given fp32 logits when logits_in != NULL), its top-k and gate weights, its
 * k expert outputs and their weighted sum in ascending expert index.  The
 * token's selections and weights are written to idx_out/w_out when given.
 */
int orc_forward_tokens(const orc_experts* X, const void* x, int x_dtype, const float* wg, const float* bias,
                       const float* logits_in, int T, int k, const int32_t* tokens, int ntok, double* y,
                       int32_t* idx_out, float* w_out, uint64_t* ops3) {
  if (check_experts(X) || T < 0 || k < 1 || k > X->E || X->E > ORC_MAX_E) return -1;
  const int m = X->m, p = X->p, E = X->E;
  int bad = 0;
  uint64_t o0 = 0, o1 = 0, o2 = 0;
#pragma omp parallel reduction(+ : o0, o1, o2) reduction(| : bad)
  {
    double* g = (double*)malloc(sizeof(double) * (size_t)p);
    double* u = (double*)malloc(sizeof(double) * (size_t)p);
    double* xr = (double*)malloc(sizeof(double) * (size_t)m);
    double* o = (double*)malloc(sizeof(double) * (size_t)m);
    double* xq = (double*)malloc(sizeof(double) * (size_t)m);
    if (!g || !u || !xr || !o || !xq) bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < ntok; ++i) {
      if (bad) continue;
      const int t = tokens[i];
      if (t < 0 || t >= T) { bad = 1; continue; }
      float lg[ORC_MAX_E];
      int32_t sel[ORC_MAX_E];
      float wt[ORC_MAX_E];
      if (logits_in) {
        for (int e = 0; e < E; ++e) lg[e] = logits_in[(int64_t)t * E + e];
      } else {
        orc_router_logits((const char*)x + (int64_t)t * m * (x_dtype == ORC_F32 ? 4 : 2), x_dtype, wg, bias, 1, m,
                          E, lg);
      }
      orc_topk(lg, 1, E, k, sel, wt);
      for (int c = 0; c < m; ++c) xr[c] = act_at(x, x_dtype, (int64_t)t * m + c);
      int slot[ORC_MAX_E];
      ascending_slots(sel, k, slot);
      double* yt = y + (int64_t)i * m;
      for (int c = 0; c < m; ++c) yt[c] = 0.0;
      uint64_t ops[3] = {0, 0, 0};
      for (int s = 0; s < k; ++s) {
        const int j = slot[s];
        expert_row(X, sel[j], xr, g, u, o, xq, ops);
        for (int c = 0; c < m; ++c) yt[c] += (double)wt[j] * o[c];
      }
      o0 += ops[0]; o1 += ops[1]; o2 += ops[2];
      if (idx_out)
        for (int j = 0; j < k; ++j) idx_out[(int64_t)i * k + j] = sel[j];
      if (w_out)
        for (int j = 0; j < k; ++j) w_out[(int64_t)i * k + j] = wt[j];
    }
    free(g); free(u); free(xr); free(o); free(xq);
  }
  if (ops3) { ops3[0] += o0; ops3[1] += o1; ops3[2] += o2; }
  return bad ? -1 : 0;
}

/* ---- dense brute force (tiny inputs) ------------------------------------ */

/*
 * y[t] = sum_{e=0}^{E-1} G[t][e] * FFN_e(x_t), with G[t][e] = w[t][j] where
 * idx[t][j] == e and 0 otherwise: every expert runs on every token and the
 * gates mask the sum.  Equal to the routed result when the routed sum runs in
 * ascending expert index.
 */
int orc_dense_masked(const orc_experts* X, const void* x, int x_dtype, const int32_t* idx, const float* w, int T,
                     int k, double* y) {
  if (check_experts(X) || T < 0 || k < 1 || k > X->E) return -1;
  const int m = X->m, p = X->p, E = X->E;
  double* g = (double*)malloc(sizeof(double) * (size_t)p);
  double* u = (double*)malloc(sizeof(double) * (size_t)p);
  double* xr = (double*)malloc(sizeof(double) * (size_t)m);
  double* o = (double*)malloc(sizeof(double) * (size_t)m);
  double* xq = (double*)malloc(sizeof(double) * (size_t)m);
  if (!g || !u || !xr || !o || !xq) { free(g); free(u); free(xr); free(o); free(xq); return -1; }
  uint64_t ops[3] = {0, 0, 0};
  for (int t = 0; t < T; ++t) {
    for (int c = 0; c < m; ++c) xr[c] = act_at(x, x_dtype, (int64_t)t * m + c);
    double* yt = y + (int64_t)t * m;
    for (int c = 0; c < m; ++c) yt[c] = 0.0;
    for (int e = 0; e < E; ++e) {
      double gate = 0.0;
      for (int j = 0; j < k; ++j)
        if (idx[(int64_t)t * k + j] == e) gate = (double)w[(int64_t)t * k + j];
      expert_row(X, e, xr, g, u, o, xq, ops);
      for (int c = 0; c < m; ++c) yt[c] += gate * o[c];
    }
  }
  free(g); free(u); free(xr); free(o); free(xq);
  return 0;
}

/* Threads the parallel loops above use (1 without OpenMP). */
int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the threads of later parallel loops (n >= 1; ignored without OpenMP). */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
