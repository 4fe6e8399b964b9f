/*
 * Seeded synthetic inputs for one MoE layer.
 *
 * This file only produces input data (activations, router weights, expert
 * weights, their int8 quantisation).  It contains none of the MoE layer's
 * arithmetic; both the CPU oracle and the GPU path read what it writes.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used in counter form: the
 * i-th output of a stream whose state starts at s is mix(s + (i+1)*gamma), so
 * every element can be produced independently and in parallel.
 * Normal deviates: Box-Muller on pairs of 53-bit uniforms, in double.
 * Each tensor has its own stream, s = seed * 2^32 + tensor_id.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* i-th (0-based) output of the SplitMix64 sequence whose state starts at s. */
uint64_t synth_splitmix64_at(uint64_t s, uint64_t i) {
  return sm64_mix(s + (i + 1) * SM64_GAMMA);
}

static inline uint64_t stream_seed(uint64_t seed, uint32_t tensor_id) {
  return (seed << 32) + (uint64_t)tensor_id;
}

/* Standard normal deviate number i of a stream (Box-Muller, double). */
double synth_normal_at(uint64_t s, uint64_t i) {
  const uint64_t pair = i >> 1;
  const uint64_t z1 = synth_splitmix64_at(s, 2 * pair);
  const uint64_t z2 = synth_splitmix64_at(s, 2 * pair + 1);
  const double u1 = (double)((z1 >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
  const double u2 = (double)(z2 >> 11) * 0x1.0p-53;       /* [0, 1) */
  const double r = sqrt(-2.0 * log(u1));
  const double th = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(th) : r * cos(th);
}

/* fp32 -> bf16 bit pattern, round to nearest even; NaN stays a quiet NaN. */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint16_t synth_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }

/* out[i] = (float)(sigma * N_i) for i < n. */
void synth_fill_normal_f32(uint64_t seed, uint32_t tensor_id, double sigma, int64_t n, float* out) {
  const uint64_t s = stream_seed(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(sigma * synth_normal_at(s, (uint64_t)i));
}

/* out[i] = bf16_rne((float)(sigma * N_i)) for i < n. */
void synth_fill_normal_bf16(uint64_t seed, uint32_t tensor_id, double sigma, int64_t n, uint16_t* out) {
  const uint64_t s = stream_seed(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)(sigma * synth_normal_at(s, (uint64_t)i)));
}

/*
 * Symmetric per-output-channel integer quantisation of a freshly generated
 * weight tensor W[E][K][N] ~ N(0, sigma^2) (fp32 values of the same stream as
 * synth_fill_normal_f32), to qmax = 127 (int8) or 7 (int4): for every expert
 * e and column n,
 *   s[e][n] = max_k |W[e][k][n]| / qmax      (fp32)
 *   q[e][k][n] = clamp(nearbyint(W / s), -qmax, qmax)   (W / s in double,
 *                round half to even), q = 0 where s == 0.
 * Quantisation is part of building the synthetic layer; the layer itself
 * then computes with q * s.
 */
int synth_fill_intq_quant(uint64_t seed, uint32_t tensor_id, double sigma, int64_t E, int64_t K, int64_t N,
                          int qmax, int8_t* q, float* scale) {
  if (qmax < 1 || qmax > 127) return -1;
  const uint64_t s = stream_seed(seed, tensor_id);
  float* w = (float*)malloc((size_t)(K * N) * sizeof(float));
  if (!w) return -1;
  for (int64_t e = 0; e < E; ++e) {
    const uint64_t base = (uint64_t)(e * K * N);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < K * N; ++i) w[i] = (float)(sigma * synth_normal_at(s, base + (uint64_t)i));
    float* se = scale + e * N;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      float mx = 0.0f;
      for (int64_t k = 0; k < K; ++k) {
        const float a = fabsf(w[k * N + n]);
        if (a > mx) mx = a;
      }
      se[n] = mx / (float)qmax;
    }
    int8_t* qe = q + e * K * N;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
      for (int64_t n = 0; n < N; ++n) {
        const float sc = se[n];
        double v = 0.0;
        if (sc != 0.0f) {
          v = nearbyint((double)w[k * N + n] / (double)sc);
          if (v > qmax) v = qmax;
          if (v < -qmax) v = -qmax;
        }
        qe[k * N + n] = (int8_t)v;
      }
    }
  }
  free(w);
  return 0;
}

int synth_fill_int8_quant(uint64_t seed, uint32_t tensor_id, double sigma, int64_t E, int64_t K, int64_t N,
                          int8_t* q, float* scale) {
  return synth_fill_intq_quant(seed, tensor_id, sigma, E, K, N, 127, q, scale);
}

/* ---- 8-bit and 4-bit float weights ---------------------------------------
 * Encoders used only to build synthetic quantised layers (the formats'
 * decoders belong to the oracle and the kernels).  Both round to nearest,
 * ties to the code with an even mantissa bit.
 */

/* |v| -> OCP E4M3 magnitude code (7 bits), v finite and |v| <= 448. */
static uint8_t e4m3_encode_mag(double a) {
  if (a < ldexp(1.0, -6)) {  /* subnormal range: m * 2^-9, m in 0..8 (8 is the smallest normal, code 8) */
    return (uint8_t)nearbyint(a / ldexp(1.0, -9));
  }
  int ex;
  const double fr = frexp(a, &ex); /* a = fr * 2^ex, fr in [0.5, 1) */
  int e = ex - 1;                  /* a = (2 fr) * 2^e, 2 fr in [1, 2) */
  int m = (int)nearbyint((2.0 * fr - 1.0) * 8.0);
  if (m == 8) {
    m = 0;
    e += 1;
  }
  int code = ((e + 7) << 3) | m;
  if (code > 0x7E) code = 0x7E; /* 448 */
  return (uint8_t)code;
}

/*
 * Per-output-channel fp8 quantisation of W[E][K][N] ~ N(0, sigma^2) (the
 * fp32 stream of synth_fill_normal_f32): s[e][n] = max_k |W| / 448 (fp32) and
 * code = E4M3 of W / s (in double, round half to even), so each column's
 * largest magnitude lands on 448; code 0 where s == 0.
 */
int synth_fill_fp8_quant(uint64_t seed, uint32_t tensor_id, double sigma, int64_t E, int64_t K, int64_t N,
                         uint8_t* q, float* scale) {
  const uint64_t s = stream_seed(seed, tensor_id);
  float* w = (float*)malloc((size_t)(K * N) * sizeof(float));
  if (!w) return -1;
  for (int64_t e = 0; e < E; ++e) {
    const uint64_t base = (uint64_t)(e * K * N);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < K * N; ++i) w[i] = (float)(sigma * synth_normal_at(s, base + (uint64_t)i));
    float* se = scale + e * N;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      float mx = 0.0f;
      for (int64_t k = 0; k < K; ++k) {
        const float a = fabsf(w[k * N + n]);
        if (a > mx) mx = a;
      }
      se[n] = mx / 448.0f;
    }
    uint8_t* qe = q + e * K * N;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
      for (int64_t n = 0; n < N; ++n) {
        const float sc = se[n];
        uint8_t c = 0;
        if (sc != 0.0f) {
          double v = (double)w[k * N + n] / (double)sc;
          if (v > 448.0) v = 448.0;
          if (v < -448.0) v = -448.0;
          c = e4m3_encode_mag(fabs(v));
          if (v < 0.0) c |= 0x80;
        }
        qe[k * N + n] = c;
      }
    }
  }
  free(w);
  return 0;
}

/* |v| -> E2M1 magnitude code (3 bits), saturating at 6; ties to the even code. */
static uint8_t e2m1_encode_mag(double a) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  if (a >= 6.0) return 7;
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    const double d = fabs(a - mag[c]), db = fabs(a - mag[best]);
    if (d < db || (d == db && (c & 1) == 0)) best = c;
  }
  return (uint8_t)best;
}

/*
 * MXFP4 quantisation of W[E][K][N] ~ N(0, sigma^2) (the fp32 stream of
 * synth_fill_normal_f32) in blocks of 32 consecutive k of one column (the OCP
 * MX block): the block's shared exponent is X = floor(log2(max |W|)) - 2 (2
 * being the largest E2M1 exponent), stored as E8M0 code X + 127 (127, scale
 * 1, for an all-zero block); each element is the E2M1 code of W / 2^X, round
 * to nearest even, saturated at 6.  codes: one per byte, [E][K][N];
 * scales: [E][K/32][N].  K must be a multiple of 32.
 */
int synth_fill_mxfp4_quant(uint64_t seed, uint32_t tensor_id, double sigma, int64_t E, int64_t K, int64_t N,
                           uint8_t* q, uint8_t* scale) {
  if (K % 32) return -1;
  const uint64_t s = stream_seed(seed, tensor_id);
  float* w = (float*)malloc((size_t)(K * N) * sizeof(float));
  if (!w) return -1;
  for (int64_t e = 0; e < E; ++e) {
    const uint64_t base = (uint64_t)(e * K * N);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < K * N; ++i) w[i] = (float)(sigma * synth_normal_at(s, base + (uint64_t)i));
    uint8_t* qe = q + e * K * N;
    uint8_t* se = scale + e * (K / 32) * N;
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < K / 32; ++g) {
      for (int64_t n = 0; n < N; ++n) {
        float mx = 0.0f;
        for (int64_t k = g * 32; k < g * 32 + 32; ++k) {
          const float a = fabsf(w[k * N + n]);
          if (a > mx) mx = a;
        }
        int X = 0;
        if (mx > 0.0f) {
          int ex;
          (void)frexp((double)mx, &ex); /* mx = fr * 2^ex, fr in [0.5, 1): floor(log2 mx) = ex - 1 */
          X = ex - 1 - 2;
          if (X < -126) X = -126;
          if (X > 127) X = 127;
        }
        se[g * N + n] = (uint8_t)(X + 127);
        for (int64_t k = g * 32; k < g * 32 + 32; ++k) {
          const double v = (double)w[k * N + n] / ldexp(1.0, X);
          uint8_t c = e2m1_encode_mag(fabs(v));
          if (v < 0.0) c |= 8;
          qe[k * N + n] = c;
        }
      }
    }
  }
  free(w);
  return 0;
}
