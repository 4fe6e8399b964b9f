/*
 * Drives the CPU oracle and the input generator through every entry point on
 * small layers of every weight kind, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  It checks nothing
 * numerically (the pins do that): the sanitizers report any out-of-bounds
 * access, leak or undefined operation, and the exit status says whether the
 * calls succeeded.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

void synth_fill_normal_f32(uint64_t seed, uint32_t tensor_id, double sigma, int64_t n, float* out);
void synth_fill_normal_bf16(uint64_t seed, uint32_t tensor_id, double sigma, int64_t n, uint16_t* out);
int synth_fill_int8_quant(uint64_t seed, uint32_t tensor_id, double sigma, int64_t E, int64_t K, int64_t N,
                          int8_t* q, float* scale);
int synth_fill_intq_quant(uint64_t seed, uint32_t tensor_id, double sigma, int64_t E, int64_t K, int64_t N, int qmax,
                          int8_t* q, float* scale);
int synth_fill_fp8_quant(uint64_t seed, uint32_t tensor_id, double sigma, int64_t E, int64_t K, int64_t N,
                         uint8_t* q, float* scale);
int synth_fill_mxfp4_quant(uint64_t seed, uint32_t tensor_id, double sigma, int64_t E, int64_t K, int64_t N,
                           uint8_t* q, uint8_t* scale);

static int bad = 0;
#define OK(call)                                              \
  do {                                                        \
    if ((call) != 0) {                                        \
      fprintf(stderr, "call failed: %s (line %d)\n", #call, __LINE__); \
      bad = 1;                                                \
    }                                                         \
  } while (0)

static void layer(int dtype, int kind, int x_bf16) {
  const int T = 7, m = 64, p = 96, E = 5, k = 2;
  const int nmat = kind == ORC_SWIGLU ? 3 : 2;
  void* w[3] = {NULL, NULL, NULL};
  void* s[3] = {NULL, NULL, NULL};
  for (int i = 0; i < nmat; ++i) {
    const int K = i == nmat - 1 ? p : m, N = i == nmat - 1 ? m : p;
    const size_t n = (size_t)E * K * N;
    switch (dtype) {
      case ORC_F32: w[i] = malloc(n * 4); synth_fill_normal_f32(3, 3 + i, 0.05, (int64_t)n, w[i]); break;
      case ORC_BF16: w[i] = malloc(n * 2); synth_fill_normal_bf16(3, 3 + i, 0.05, (int64_t)n, w[i]); break;
      case ORC_I8:
      case ORC_I8A8:
        w[i] = malloc(n); s[i] = malloc((size_t)E * N * 4);
        OK(i % 2 ? synth_fill_intq_quant(3, 3 + i, 0.05, E, K, N, 7, w[i], s[i])
                 : synth_fill_int8_quant(3, 3 + i, 0.05, E, K, N, w[i], s[i]));
        break;
      case ORC_FP8:
      case ORC_FP8A8:
        w[i] = malloc(n); s[i] = malloc((size_t)E * N * 4);
        OK(synth_fill_fp8_quant(3, 3 + i, 0.05, E, K, N, w[i], s[i]));
        break;
      default:
        w[i] = malloc(n); s[i] = malloc((size_t)E * (K / 32) * N);
        OK(synth_fill_mxfp4_quant(3, 3 + i, 0.05, E, K, N, w[i], s[i]));
        break;
    }
  }
  orc_experts X = {m, p, E, kind, dtype, w[0], kind == ORC_SWIGLU ? w[1] : NULL, w[nmat - 1],
                   s[0], kind == ORC_SWIGLU ? s[1] : NULL, s[nmat - 1]};
  void* x = malloc((size_t)T * m * 4);
  if (x_bf16) synth_fill_normal_bf16(3, 0, 1.0, (int64_t)T * m, x);
  else synth_fill_normal_f32(3, 0, 1.0, (int64_t)T * m, x);
  const int xdt = x_bf16 ? ORC_BF16 : ORC_F32;
  float* wg = malloc((size_t)m * E * 4);
  synth_fill_normal_f32(3, 1, 0.05, (int64_t)m * E, wg);
  float bias[5] = {0.1f, -0.2f, 0.0f, 0.3f, -0.1f};
  float* logits = malloc((size_t)T * E * 4);
  int32_t *idx = malloc((size_t)T * k * 4), *counts = malloc((size_t)E * 4), *offsets = malloc((size_t)(E + 1) * 4);
  int32_t *perm = malloc((size_t)T * k * 4), *inv = malloc((size_t)T * k * 4);
  float* tw = malloc((size_t)T * k * 4);
  OK(orc_router_logits(x, xdt, wg, bias, T, m, E, logits));
  logits[3] = NAN;
  OK(orc_topk(logits, T, E, k, idx, tw));
  OK(orc_dispatch(idx, T, E, k, counts, offsets, perm, inv));
  double* yp = malloc((size_t)T * k * m * 8);
  double* y = malloc((size_t)T * m * 8);
  double* yd = malloc((size_t)T * m * 8);
  uint64_t ops[3] = {0, 0, 0};
  OK(orc_expert_rows(&X, x, xdt, T, k, perm, offsets, NULL, 0, yp, ops));
  int32_t rows[3] = {0, 5, T * k - 1};
  OK(orc_expert_rows(&X, x, xdt, T, k, perm, offsets, rows, 3, yp, ops));
  OK(orc_combine(yp, inv, idx, tw, T, m, k, y));
  int32_t toks[3] = {6, 0, 2};
  int32_t idx3[6];
  float w3[6];
  OK(orc_forward_tokens(&X, x, xdt, wg, bias, NULL, T, k, toks, 3, y, idx3, w3, ops));
  OK(orc_dense_masked(&X, x, xdt, idx, tw, T, k, yd));
  double xr[64], o[64];
  for (int i = 0; i < m; ++i) xr[i] = 0.01 * i;
  OK(orc_expert_apply(&X, E - 1, xr, o, ops));
  double v;
  OK(orc_weight_value(w[0], s[0], dtype, E - 1, m, p, m - 1, p - 1, &v));
  float gamma[64], beta[64];
  for (int i = 0; i < m; ++i) { gamma[i] = 1.0f; beta[i] = 0.0f; }
  double* xn = malloc((size_t)T * m * 8);
  OK(orc_norm(x, xdt, T, m, ORC_NORM_LAYER, gamma, beta, 1e-5, xn));
  OK(orc_norm(x, xdt, T, m, ORC_NORM_RMS, gamma, NULL, 1e-5, xn));
  {
    uint8_t* qc = malloc((size_t)T * m);
    float* qs = malloc((size_t)T * 4);
    OK(orc_quant_rows_e4m3(x, xdt, T, m, xn, qc, qs));
    OK(orc_quant_rows_i8(x, xdt, T, m, xn, (int8_t*)qc, qs));
    OK(orc_e4m3_encode(tw, (int64_t)T * k, qc));
    free(qc);
    free(qs);
  }
  /* rejected arguments return -1 without touching memory */
  if (orc_topk(logits, T, E, E + 1, idx, tw) != -1 || orc_dispatch(idx, T, 0, k, counts, offsets, perm, inv) != -1) bad = 1;
  for (int i = 0; i < 3; ++i) { free(w[i]); free(s[i]); }
  free(x); free(wg); free(logits); free(idx); free(counts); free(offsets); free(perm); free(inv); free(tw);
  free(yp); free(y); free(yd); free(xn);
}

int main(void) {
  const int dtypes[7] = {ORC_F32, ORC_BF16, ORC_I8, ORC_FP8, ORC_MXFP4, ORC_FP8A8, ORC_I8A8};
  for (int d = 0; d < 7; ++d)
    for (int kind = 0; kind < 2; ++kind) layer(dtypes[d], kind, dtypes[d] != ORC_F32);
  if (bad) return 1;
  printf("sanitized run ok\n");
  return 0;
}
