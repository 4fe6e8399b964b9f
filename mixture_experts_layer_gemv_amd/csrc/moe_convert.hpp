// Exact conversions of packed integer weights to bf16 MFMA operands, shared
// by the decode kernels and the grouped GEMM.  The integer kinds keep their
// per-output-channel scale for the epilogue, so a weight enters the product
// as its integer value (int8) or as that value plus a constant (int4, see
// below), both exact in bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_kernels.hpp"

namespace moe {

typedef uint32_t cvt_u32x4_t __attribute__((ext_vector_type(4)));

// 8 signed bytes (two dwords) -> 8 bf16.  |q| <= 128 is exact in bf16, so the
// fp32 value's upper half is the bf16 pattern.
__device__ __forceinline__ bf16x8_t i8x8_to_bf16(uint32_t lo, uint32_t hi) {
  cvt_u32x4_t r;
  const uint32_t d[2] = {lo, hi};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const float f0 = (float)(signed char)(d[q]);
    const float f1 = (float)(signed char)(d[q] >> 8);
    const float f2 = (float)(signed char)(d[q] >> 16);
    const float f3 = (float)(signed char)(d[q] >> 24);
    r[2 * q] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    r[2 * q + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
  }
  return __builtin_bit_cast(bf16x8_t, r);
}

// 8 int4 weights stored offset by 8 (u = q + 8; values 0-3 in the low
// nibbles of bytes 0-3, values 4-7 in the high nibbles) -> the 8 bf16 values
// 128 + u, exactly: the bf16 pattern of 128 (0x4300) leaves the value's
// integer part to its 7 mantissa bits, so each value is its nibble as the low
// byte under a high byte of 0x43.  After masking, one byte permute per pair
// takes two nibble bytes and two 0x43 bytes; the products' constant part
// 136 * sum(x) is removed after the reduction.
__device__ __forceinline__ bf16x8_t u4x8_to_bf16_biased(uint32_t d) {
  const uint32_t t0 = d & 0x0F0F0F0Fu, t1 = (d >> 4) & 0x0F0F0F0Fu;
  const uint32_t hi = 0x43434343u;  // (selector bytes 4-7)
  cvt_u32x4_t r;
  r[0] = __builtin_amdgcn_perm(hi, t0, 0x04010400u);  // values 0, 1
  r[1] = __builtin_amdgcn_perm(hi, t0, 0x04030402u);  // values 2, 3
  r[2] = __builtin_amdgcn_perm(hi, t1, 0x04010400u);  // values 4, 5
  r[3] = __builtin_amdgcn_perm(hi, t1, 0x04030402u);  // values 6, 7
  return __builtin_bit_cast(bf16x8_t, r);
}
constexpr float kI4Bias = 136.0f;  // 128 from the bf16 pattern + 8 from the storage offset


// 8 OCP E4M3 codes (two dwords, byte j = value j) -> 8 bf16, exactly (every
// E4M3 value is a bf16 value): the hardware conversion of two codes at a
// time, scale 1 (the per-channel scale is applied in the epilogue).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  cvt_u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return __builtin_bit_cast(bf16x8_t, r);
}

// 8 E2M1 codes (one dword, byte b holding values 2b in its low and 2b+1 in
// its high nibble) times their block's scale -> 8 bf16: the hardware
// conversion of one byte at a time with the E8M0 scale applied, exact while
// the scaled values stay inside bf16's normal range (block exponents
// 2^-100 .. 2^100 leave a wide margin).
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t d, float scale) {
  cvt_u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3));
  return __builtin_bit_cast(bf16x8_t, r);
}

// The E8M0 exponent E in byte h of a scale dword as the fp32 2^(E - 127)
// (E in 1 .. 254).
__device__ __forceinline__ float e8m0_at(uint32_t d, int h) { return __uint_as_float(((d >> (8 * h)) & 255u) << 23); }

// Weight kinds of the kernel variants, by their code qb: 0 bf16, 8 int8,
// 9 fp8 (E4M3), 4 int4, 5 MXFP4 (E2M1 with E8M0 block scales).  A lane's
// 16-byte load of packed weights covers q_ah(qb) MFMA K steps of 32.
constexpr int q_bits(int qb) { return qb >= 8 ? 8 : (qb >= 4 ? 4 : 16); }
constexpr int q_ah(int qb) { return qb >= 8 ? 2 : (qb >= 4 ? 4 : 1); }
// per-output-channel scales applied in the epilogue (int8, fp8, int4)
constexpr bool q_chan_scale(int qb) { return qb == 8 || qb == 9 || qb == 4; }

// ---- 8-bit activations ------------------------------------------------------------

// The value of an E4M3 magnitude code.
__device__ __forceinline__ float e4m3_mag(uint32_t c) {
  const int ex = (int)(c >> 3), mt = (int)(c & 7);
  return ex == 0 ? ldexpf((float)mt, -9) : ldexpf((float)(8 + mt), ex - 10);
}

// The power-of-two exponent X of a row's activation scale: the smallest
// integer with amax <= qmax * 2^X, qmax = 448 (E4M3) or 127 (int8), from the
// exact binary form amax = f * 2^e, f in [1, 2): X = e - 8 when f <= 1.75
// (E4M3), e - 6 when f <= 127/64 (int8), else one more.  0 for amax = 0.
template <bool INT8>
__device__ __forceinline__ int act_scale_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e2;
  const float f = 2.0f * frexpf(amax, &e2);  // amax = f * 2^(e2 - 1)
  return INT8 ? (e2 - 1) - (f <= 127.0f / 64.0f ? 6 : 5) : (e2 - 1) - (f <= 1.75f ? 8 : 7);
}

// Quantises eight bf16 activations of a row (one 16-byte load) with the row's
// scale 2^X: their codes (bytes in element order; E4M3 with the sign in bit
// 7, or int8 two's complement) and, with VALUES, the quantised values as
// bf16.  The division by 2^X is exact.  E4M3 codes come from the hardware
// conversion (round to nearest, ties to even, onto the OCP E4M3 grid; |v| <=
// 448 never saturates), which was checked against a plain encoder of the
// grid on the GPU for every bf16 input of magnitude <= 448, both signs; int8
// codes round the quotient half to even (|q| <= 127).  A value is the code's
// number times 2^X with the input's sign (zero included): at most seven
// significant bits, so bf16 holds it exactly.
template <bool INT8, bool VALUES>
__device__ __forceinline__ void quant8(const uint32_t (&w)[4], int X, uint32_t (&q)[4], uint32_t (&c)[2]) {
  c[0] = c[1] = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t b0 = w[j] & 0xFFFFu, b1 = w[j] >> 16;
    uint32_t code2;
    if constexpr (INT8) {
      // the signed quotient rounded (a rounded -0 keeps its sign for the value)
      const float r0 = rintf(ldexpf(__uint_as_float(b0 << 16), -X));
      const float r1 = rintf(ldexpf(__uint_as_float(b1 << 16), -X));
      code2 = ((uint32_t)(int)r0 & 0xFFu) | (((uint32_t)(int)r1 & 0xFFu) << 8);
      if constexpr (VALUES)
        q[j] = (__float_as_uint(ldexpf(r0, X)) >> 16) | (__float_as_uint(ldexpf(r1, X)) & 0xFFFF0000u);
    } else {
      code2 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(__uint_as_float(b0 << 16), -X),
                                                        ldexpf(__uint_as_float(b1 << 16), -X), 0, false) &
              0xFFFFu;
      if constexpr (VALUES) {
        const float v0 = ldexpf(e4m3_mag(code2 & 0x7Fu), X), v1 = ldexpf(e4m3_mag((code2 >> 8) & 0x7Fu), X);
        q[j] = ((__float_as_uint(v0) >> 16) | (b0 & 0x8000u)) | (((__float_as_uint(v1) >> 16) | (b1 & 0x8000u)) << 16);
      }
    }
    c[j >> 1] |= code2 << (16 * (j & 1));
  }
}

}  // namespace moe
