/*
 * CPU oracle for one MoE-layer forward pass -- TEST INFRASTRUCTURE ONLY.
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load it.  It shares no code, header or constant with the HIP library.
 * Definitions and citations: moe_oracle.c.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#define ORC_MAX_E 64

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_I8 = 2, ORC_FP8 = 3, ORC_MXFP4 = 4, ORC_FP8A8 = 5, ORC_I8A8 = 6 };
enum { ORC_RELU = 0, ORC_SWIGLU = 1 };

/* Expert weights in canonical row-major layout:
 * w1 (ReLU MLP W1, or SwiGLU gate) [E][m][p], w3 (SwiGLU up) [E][m][p],
 * w2 (second / down) [E][p][m].  Scales: int8 and fp8 fp32 s1, s3 [E][p],
 * s2 [E][m]; MXFP4 uint8 E8M0 s1, s3 [E][m/32][p], s2 [E][p/32][m].
 * ORC_FP8A8: fp8 weights as ORC_FP8, and each token's input to the first
 * projection quantized to E4M3 first (orc_quant_rows_e4m3). */
typedef struct {
  int m, p, E, kind, w_dtype;
  const void *w1, *w3, *w2;
  const void *s1, *s3, *s2;
} orc_experts;

/* One decoded weight (e, k, n) of a [E][K][N] projection in dtype, with its
 * scales s (as in orc_experts). */
int orc_weight_value(const void* w, const void* s, int dtype, int64_t e, int64_t K, int64_t N, int64_t k, int64_t n,
                     double* out);

/* E4M3 codes of fp32 values (round to nearest even, magnitudes of 448 and
 * above saturating to 448). */
int orc_e4m3_encode(const float* v, int64_t n, uint8_t* codes);
/* Per-row E4M3 quantisation of T rows of m activations: scale s = 2^X, the
 * smallest power of two with amax <= 448 s; out = e4m3(code) * s (double);
 * codes and scales when non-NULL. */
int orc_quant_rows_e4m3(const void* x, int x_dtype, int T, int m, double* out, uint8_t* codes, float* scales);
/* Per-row int8 quantisation: scale s = 2^X, the smallest power of two with
 * amax <= 127 s; q = round-to-nearest-even(x / s); out = q * s. */
int orc_quant_rows_i8(const void* x, int x_dtype, int T, int m, double* out, int8_t* codes, float* scales);

int orc_router_logits(const void* x, int x_dtype, const float* wg, const float* bias, int T, int m, int E,
                      float* logits);
int orc_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w);
int orc_dispatch(const int32_t* idx, int T, int E, int k, int32_t* counts, int32_t* offsets, int32_t* perm,
                 int32_t* inv_perm);
int orc_expert_apply(const orc_experts* X, int e, const double* x, double* o, uint64_t* ops3);
int orc_expert_rows(const orc_experts* X, const void* x, int x_dtype, int T, int k, const int32_t* perm,
                    const int32_t* offsets, const int32_t* rows, int nrows, double* out, uint64_t* ops3);
int orc_combine(const double* y_perm, const int32_t* inv_perm, const int32_t* idx, const float* w, int T, int m,
                int k, double* y);
int orc_forward_tokens(const orc_experts* X, const void* x, int x_dtype, const float* wg, const float* bias,
                       const float* logits_in, int T, int k, const int32_t* tokens, int ntok, double* y,
                       int32_t* idx_out, float* w_out, uint64_t* ops3);
int orc_dense_masked(const orc_experts* X, const void* x, int x_dtype, const int32_t* idx, const float* w, int T,
                     int k, double* y);

/* Norm before the layer: ORC_NORM_LAYER (mean and biased variance over the
 * row) or ORC_NORM_RMS (root mean square); out in double. */
enum { ORC_NORM_LAYER = 1, ORC_NORM_RMS = 2 };
int orc_norm(const void* x, int x_dtype, int T, int m, int kind, const float* gamma, const float* beta, double eps,
             double* out);

int orc_max_threads(void);
void orc_set_threads(int n);

#endif
