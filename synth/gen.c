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
