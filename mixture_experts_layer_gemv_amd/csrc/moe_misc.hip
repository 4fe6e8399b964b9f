// Supporting kernels: init-time weight packing, the fp32 expert FFN, the
// standalone weighted combine and small elementwise passes.
#include "moe_convert.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

// ---- packing (run once in moe_weights_create) ------------------------------

// One thread writes one lane's 16 bytes of one 1 KiB block (layout described
// in moe_kernels.hpp).  Reads are strided; this runs once per layer.
__global__ __launch_bounds__(256) void k_pack_bf16(const uint16_t* __restrict__ src, uint4* __restrict__ dst, int E,
                                                   int K, int N, int G, int g) {
  const int NB = N / 16, U = K / 32;
  const size_t total = (size_t)E * NB * U * 64;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63);
    size_t rest = i >> 6;
    const int u = (int)(rest % U);
    rest /= U;
    const int nb = (int)(rest % NB);
    const int e = (int)(rest / NB);
    const int n = nb * 16 + (lane & 15);
    const int k0 = u * 32 + 8 * (lane >> 4);
    const uint16_t* s = src + ((size_t)e * K + k0) * N + n;
    uint32_t d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = (uint32_t)s[(size_t)(2 * j) * N] | ((uint32_t)s[(size_t)(2 * j + 1) * N] << 16);
    dst[((((size_t)e * NB + nb) * U + u) * G + g) * 64 + lane] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

__global__ __launch_bounds__(256) void k_pack_i8(const int8_t* __restrict__ src, uint4* __restrict__ dst, int E,
                                                 int K, int N, int G, int g) {
  const int NB = N / 16, U = K / 64;
  const size_t total = (size_t)E * NB * U * 64;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63);
    size_t rest = i >> 6;
    const int u = (int)(rest % U);
    rest /= U;
    const int nb = (int)(rest % NB);
    const int e = (int)(rest / NB);
    const int n = nb * 16 + (lane & 15);
    uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kk = u * 64 + 32 * (j >> 3) + 8 * (lane >> 4) + (j & 7);
      const uint32_t byte = (uint8_t)src[((size_t)e * K + kk) * N + n];
      d[j >> 2] |= byte << (8 * (j & 3));
    }
    dst[((((size_t)e * NB + nb) * U + u) * G + g) * 64 + lane] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

// int4 (held one per int8, in [-8, 7]): 128 k per unit; value j of a lane's
// 32 is k = 32 (j / 8) + 8 (lane / 16) + j % 8, in dword j / 8: values 0-3 of
// a dword in the low nibbles of its bytes 0-3, values 4-7 in the high
// nibbles, each stored offset by 8 (q + 8 in [0, 15]).
__global__ __launch_bounds__(256) void k_pack_i4(const int8_t* __restrict__ src, uint4* __restrict__ dst, int E,
                                                 int K, int N, int G, int g) {
  const int NB = N / 16, U = K / 128;
  const size_t total = (size_t)E * NB * U * 64;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63);
    size_t rest = i >> 6;
    const int u = (int)(rest % U);
    rest /= U;
    const int nb = (int)(rest % NB);
    const int e = (int)(rest / NB);
    const int n = nb * 16 + (lane & 15);
    uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int kk = u * 128 + 32 * (j >> 3) + 8 * (lane >> 4) + (j & 7);
      const uint32_t nib = (uint32_t)(src[((size_t)e * K + kk) * N + n] + 8) & 0xFu;
      d[j >> 3] |= nib << (8 * (j & 3) + 4 * ((j >> 2) & 1));
    }
    dst[((((size_t)e * NB + nb) * U + u) * G + g) * 64 + lane] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

// MXFP4 codes (one per byte, low nibble): 128 k per unit; value j of a
// lane's 32 is k = 32 (j / 8) + 8 (lane / 16) + j % 8, in dword j / 8, byte
// (j % 8) / 2, the low nibble for even j (the order the hardware conversion
// takes a byte's two values in).
__global__ __launch_bounds__(256) void k_pack_fp4(const uint8_t* __restrict__ src, uint4* __restrict__ dst, int E,
                                                  int K, int N, int G, int g) {
  const int NB = N / 16, U = K / 128;
  const size_t total = (size_t)E * NB * U * 64;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63);
    size_t rest = i >> 6;
    const int u = (int)(rest % U);
    rest /= U;
    const int nb = (int)(rest % NB);
    const int e = (int)(rest / NB);
    const int n = nb * 16 + (lane & 15);
    uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int kk = u * 128 + 32 * (j >> 3) + 8 * (lane >> 4) + (j & 7);
      const uint32_t nib = (uint32_t)src[((size_t)e * K + kk) * N + n] & 0xFu;
      d[j >> 3] |= nib << (8 * ((j & 7) >> 1) + 4 * (j & 1));
    }
    dst[((((size_t)e * NB + nb) * U + u) * G + g) * 64 + lane] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

// MXFP4 block scales X[e][K/32][N] -> per (expert, tile, unit, stream) 16
// dwords, dword c = the four E8M0 bytes of column nb*16 + c for the unit's
// 32-k steps 0..3.
__global__ __launch_bounds__(256) void k_pack_mx_scales(const uint8_t* __restrict__ src, uint32_t* __restrict__ dst,
                                                        int E, int K, int N, int G, int g) {
  const int NB = N / 16, U = K / 128;
  const size_t total = (size_t)E * NB * U * 16;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(i & 15);
    size_t rest = i >> 4;
    const int u = (int)(rest % U);
    rest /= U;
    const int nb = (int)(rest % NB);
    const int e = (int)(rest / NB);
    const int n = nb * 16 + c;
    uint32_t d = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) d |= (uint32_t)src[((size_t)e * (K / 32) + 4 * u + h) * N + n] << (8 * h);
    dst[((((size_t)e * NB + nb) * U + u) * G + g) * 16 + c] = d;
  }
}

// MXFP4 weights expanded exactly to the packed bf16 layout of the grouped GEMM
// (prefill sizes): one thread per lane of a packed unit (128 k of one column
// stream); dword h of the unit holds the lane's eight values of 32-k step
// 4u + h, whose block scale is byte h of the column's scale dword, and they
// become the lane's 16 bytes of bf16 unit 4u + h.  E2M1 values times an E8M0
// scale are bf16 values (two significant bits).  Experts without rows (per
// offsets, when given) are skipped.
__global__ __launch_bounds__(256) void k_expand_fp4(const uint4* __restrict__ src, const uint32_t* __restrict__ sc,
                                                    uint4* __restrict__ dst, const int32_t* __restrict__ offsets,
                                                    int E, int K, int N, int G) {
  const int NB = N / 16, U = K / 128;
  const size_t total = (size_t)E * NB * U * G * 64;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63);
    size_t rest = i >> 6;  // (((e * NB + nb) * U + u) * G + g)
    const int g = (int)(rest % G);
    const size_t eu = rest / G;  // ((e * NB + nb) * U + u)
    const int u = (int)(eu % U);
    const int e = (int)(eu / U / NB);
    if (offsets && offsets[e + 1] == offsets[e]) continue;
    const uint4 q = src[i];
    const uint32_t d = sc[rest * 16 + (lane & 15)];
    const size_t o = ((eu / U * (size_t)(4 * U) + 4 * (size_t)u) * G + g) * 64 + lane;  // bf16 unit 4u of the same tile
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int h = 0; h < 4; ++h)
      dst[o + (size_t)h * G * 64] = __builtin_bit_cast(uint4, fp4x8_to_bf16(w[h], e8m0_at(d, h)));
  }
}

// ---- fp32 expert FFN ------------------------------------------------------------
//
// True fp32 arithmetic (one fused multiply-add per term, in increasing k) for
// fp32 layers.  Block = (expert, 16-row chunk) x 256 output columns; each
// thread owns one column and up to 16 rows.  The chunk's activation rows are
// staged in LDS, kKc columns at a time (rows past the chunk's last are zero
// and never stored), so the k loop issues only the weight loads, unrolled to
// keep several in flight.

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

constexpr int kF32Rows = 16;
constexpr int kKc = 256;  // staged activation columns per round (16 KiB)

template <int EPI>
__global__ __launch_bounds__(256) void k_ffn_f32(const F32Args A) {
  constexpr int R = kF32Rows;
  __shared__ float xs[R][kKc];
  __shared__ int src_s[R];
  int e = -1, chunk = 0;
  {
    int rem = blockIdx.x;
    for (int i = 0; i < A.E; ++i) {
      const int c = A.offsets[i + 1] - A.offsets[i];
      const int nch = (c + R - 1) / R;
      if (rem < nch) {
        e = i;
        chunk = rem;
        break;
      }
      rem -= nch;
    }
  }
  if (e < 0) return;
  const int tid = threadIdx.x;
  const int n = blockIdx.y * 256 + tid;
  const bool col = n < A.N;
  const int row0 = A.offsets[e] + chunk * R;
  const int nrows = min(R, A.offsets[e + 1] - row0);
  if (tid < R) src_s[tid] = tid < nrows ? (A.gather ? A.perm[row0 + tid] / A.topk : row0 + tid) : -1;
  __syncthreads();
  constexpr bool GATED = EPI == EPI_UP_SWIGLU;
  float acc1[R], acc3[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc1[r] = acc3[r] = 0.0f;
  const float* w1 = A.w1 + (size_t)e * A.K * A.N + (col ? n : 0);
  const float* w3 = GATED ? A.w3 + (size_t)e * A.K * A.N + (col ? n : 0) : nullptr;
  for (int k0 = 0; k0 < A.K; k0 += kKc) {
    const int kc = min(kKc, A.K - k0);
    // stage rows x columns [k0, k0 + kc) (zeros past the chunk's rows)
    for (int q = tid; q < R * kKc; q += 256) {
      const int r = q / kKc, c = q - r * kKc;
      const int sr = src_s[r];
      xs[r][c] = sr >= 0 && c < kc ? A.act[(size_t)sr * A.K + k0 + c] : 0.0f;
    }
    __syncthreads();
    if (col) {
#pragma unroll 8
      for (int kk = 0; kk < kc; ++kk) {
        const float a1 = w1[(size_t)(k0 + kk) * A.N];
        const float a3 = GATED ? w3[(size_t)(k0 + kk) * A.N] : 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float xv = xs[r][kk];
          acc1[r] = fmaf(xv, a1, acc1[r]);
          if (GATED) acc3[r] = fmaf(xv, a3, acc3[r]);
        }
      }
    }
    __syncthreads();
  }
  if (!col) return;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= nrows) continue;
    const int row = row0 + r;
    if constexpr (EPI == EPI_UP_SWIGLU) {
      A.out[(size_t)row * A.N + n] = silu_f(acc1[r]) * acc3[r];
    } else if constexpr (EPI == EPI_UP_RELU) {
      A.out[(size_t)row * A.N + n] = acc1[r] > 0.0f ? acc1[r] : 0.0f;
    } else if constexpr (EPI == EPI_DOWN_ACC) {
      const int a = A.perm[row];
      unsafeAtomicAdd(A.out + (size_t)(a / A.topk) * A.N + n, A.topk_w[a] * acc1[r]);
    } else {
      A.out[(size_t)row * A.N + n] = acc1[r];
    }
  }
}

// ---- combine and elementwise ----------------------------------------------------

// y[t][c] = sum_{j<k} w[t][j] * y_perm[inv_perm[t*k+j]][c] (+ residual[t][c],
// in y's dtype, added last).  A thread takes V float4 columns of one row,
// R = m / (4 V) float4 apart (so each of its V loads is coalesced across the
// row's threads), and issues the V loads of a row slice together.
template <bool BF16, int V>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y_perm, const int32_t* __restrict__ inv,
                                                 const float* __restrict__ w, int T, int m, int k, int slices,
                                                 size_t slice_stride, const void* __restrict__ residual,
                                                 void* __restrict__ y) {
  const size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int R = m / (4 * V);  // threads per row
  if (g >= (size_t)T * R) return;
  const int t = (int)(g / R);
  const int c0 = (int)(g - (size_t)t * R) * 4;  // first column; the others 4 R apart
  float4 s[V];
#pragma unroll
  for (int v = 0; v < V; ++v) s[v] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const float* row = y_perm + (size_t)inv[(size_t)t * k + j] * m + c0;
    // the row's partial sums over the reduction slices, in slice order
    float4 acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = *reinterpret_cast<const float4*>(row + v * 4 * R);
    for (int q = 1; q < slices; ++q) {
      float4 u[V];
#pragma unroll
      for (int v = 0; v < V; ++v) u[v] = *reinterpret_cast<const float4*>(row + (size_t)q * slice_stride + v * 4 * R);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        acc[v].x += u[v].x;
        acc[v].y += u[v].y;
        acc[v].z += u[v].z;
        acc[v].w += u[v].w;
      }
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      s[v].x = fmaf(wj, acc[v].x, s[v].x);
      s[v].y = fmaf(wj, acc[v].y, s[v].y);
      s[v].z = fmaf(wj, acc[v].z, s[v].z);
      s[v].w = fmaf(wj, acc[v].w, s[v].w);
    }
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const size_t off = (size_t)t * m + c0 + v * 4 * R;
    if (residual) {
      if (BF16) {
        const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(residual) + off);
        s[v].x += bf16_to_f32((uint16_t)(r.x & 0xFFFFu));
        s[v].y += bf16_to_f32((uint16_t)(r.x >> 16));
        s[v].z += bf16_to_f32((uint16_t)(r.y & 0xFFFFu));
        s[v].w += bf16_to_f32((uint16_t)(r.y >> 16));
      } else {
        const float4 r = *reinterpret_cast<const float4*>(static_cast<const float*>(residual) + off);
        s[v].x += r.x;
        s[v].y += r.y;
        s[v].z += r.z;
        s[v].w += r.w;
      }
    }
    if (BF16) {
      const uint2 pk = make_uint2((uint32_t)f32_to_bf16(s[v].x) | ((uint32_t)f32_to_bf16(s[v].y) << 16),
                                  (uint32_t)f32_to_bf16(s[v].z) | ((uint32_t)f32_to_bf16(s[v].w) << 16));
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + off) = pk;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(y) + off) = s[v];
    }
  }
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, size_t n) {
  const size_t n4 = n / 4;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x)
    reinterpret_cast<float4*>(p)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  const size_t tail = n4 * 4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tail < n) p[tail] = 0.0f;
}

__global__ __launch_bounds__(256) void k_f32_to_bf16(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                     size_t n) {
  const size_t n4 = n / 4;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
    const float4 v = reinterpret_cast<const float4*>(src)[i];
    reinterpret_cast<uint2*>(dst)[i] = make_uint2((uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16),
                                                  (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16));
  }
  const size_t tail = n4 * 4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tail < n) dst[tail] = f32_to_bf16(src[tail]);
}

unsigned grid_for(size_t work, unsigned cap = 65536u) {
  size_t b = (work + 255) / 256;
  if (b < 1) b = 1;
  return (unsigned)(b < cap ? b : cap);
}

}  // namespace

hipError_t launch_pack_bf16(const uint16_t* src, void* dst, int E, int K, int N, int G, int g, hipStream_t s) {
  const size_t total = (size_t)E * (N / 16) * (K / 32) * 64;
  k_pack_bf16<<<grid_for(total, 1u << 20), 256, 0, s>>>(src, static_cast<uint4*>(dst), E, K, N, G, g);
  return hipGetLastError();
}

hipError_t launch_pack_i8(const int8_t* src, void* dst, int E, int K, int N, int G, int g, hipStream_t s) {
  const size_t total = (size_t)E * (N / 16) * (K / 64) * 64;
  k_pack_i8<<<grid_for(total, 1u << 20), 256, 0, s>>>(src, static_cast<uint4*>(dst), E, K, N, G, g);
  return hipGetLastError();
}

hipError_t launch_pack_i4(const int8_t* src, void* dst, int E, int K, int N, int G, int g, hipStream_t s) {
  const size_t total = (size_t)E * (N / 16) * (K / 128) * 64;
  k_pack_i4<<<grid_for(total, 1u << 20), 256, 0, s>>>(src, static_cast<uint4*>(dst), E, K, N, G, g);
  return hipGetLastError();
}

hipError_t launch_pack_fp4(const uint8_t* src, void* dst, int E, int K, int N, int G, int g, hipStream_t s) {
  const size_t total = (size_t)E * (N / 16) * (K / 128) * 64;
  k_pack_fp4<<<grid_for(total, 1u << 20), 256, 0, s>>>(src, static_cast<uint4*>(dst), E, K, N, G, g);
  return hipGetLastError();
}

hipError_t launch_expand_fp4(const void* w, const uint32_t* scales, void* dst, const int32_t* offsets, int E, int K,
                             int N, int G, hipStream_t s) {
  if (K % 128 || N % 16) return hipErrorInvalidValue;
  const size_t total = (size_t)E * (N / 16) * (K / 128) * G * 64;
  if (total == 0) return hipSuccess;
  k_expand_fp4<<<grid_for(total, 1u << 20), 256, 0, s>>>(static_cast<const uint4*>(w), scales, static_cast<uint4*>(dst),
                                                           offsets, E, K, N, G);
  return hipGetLastError();
}

hipError_t launch_pack_mx_scales(const uint8_t* src, void* dst, int E, int K, int N, int G, int g, hipStream_t s) {
  const size_t total = (size_t)E * (N / 16) * (K / 128) * 16;
  k_pack_mx_scales<<<grid_for(total, 1u << 20), 256, 0, s>>>(src, static_cast<uint32_t*>(dst), E, K, N, G, g);
  return hipGetLastError();
}

hipError_t launch_ffn_f32(const F32Args& a, hipStream_t s) {
  const dim3 grid((unsigned)a.W, (unsigned)((a.N + 255) / 256)), block(256);
  switch (a.epi) {
    case EPI_UP_SWIGLU: k_ffn_f32<EPI_UP_SWIGLU><<<grid, block, 0, s>>>(a); break;
    case EPI_UP_RELU: k_ffn_f32<EPI_UP_RELU><<<grid, block, 0, s>>>(a); break;
    case EPI_DOWN_ACC: k_ffn_f32<EPI_DOWN_ACC><<<grid, block, 0, s>>>(a); break;
    default: k_ffn_f32<EPI_DOWN_ROWS><<<grid, block, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w, int T, int m, int k,
                          int slices, size_t slice_stride, void* y, bool y_bf16, hipStream_t s,
                          const void* residual) {
  if (slices < 1 || m % 16) return hipErrorInvalidValue;
  const size_t work = (size_t)T * (m / 4);  // float4 columns
  if (work == 0) return hipSuccess;
  // four float4 per thread once there are enough rows to fill the GPU with
  // the fewer threads (prefill); one at decode sizes
  const bool wide = work >= ((size_t)1 << 20);
  const unsigned grid = (unsigned)(((wide ? work / 4 : work) + 255) / 256);
  if (wide) {
    if (y_bf16)
      k_combine<true, 4><<<grid, 256, 0, s>>>(y_perm, inv_perm, topk_w, T, m, k, slices, slice_stride, residual, y);
    else
      k_combine<false, 4><<<grid, 256, 0, s>>>(y_perm, inv_perm, topk_w, T, m, k, slices, slice_stride, residual, y);
  } else {
    if (y_bf16)
      k_combine<true, 1><<<grid, 256, 0, s>>>(y_perm, inv_perm, topk_w, T, m, k, slices, slice_stride, residual, y);
    else
      k_combine<false, 1><<<grid, 256, 0, s>>>(y_perm, inv_perm, topk_w, T, m, k, slices, slice_stride, residual, y);
  }
  return hipGetLastError();
}

// ---- fp8 activations ------------------------------------------------------------
//
// The experts of an fp8-activation layer read each token's row quantised to
// the OCP E4M3 format (sign, 4 exponent bits with bias 7, 3 mantissa bits,
// largest finite 448) with one power-of-two scale per row, in the spirit of
// the DeepSpeed-Inference summary's INT8 GeMM, which quantises its
// activations (datalearner.com, section 4).  The scale is 2^X with X the
// smallest integer such that max|x| <= 448 * 2^X, so dividing by it is exact
// and no element saturates; the product of an E4M3 value and 2^X has four
// significant bits, so bf16 holds the quantised value exactly and the decode
// kernels read it unchanged.

// One workgroup per row: the row's maximum magnitude, its scale, then the
// quantised row as bf16 values (xq) and/or as codes (xc: E4M3 with the sign
// in bit 7, or int8), each output skipped when its pointer is null.  The
// int8 form: scale 2^X, X the smallest integer with max|x| <= 127 * 2^X, q =
// x / 2^X rounded half to even (|q| <= 127); q * 2^X has seven significant
// bits, so bf16 holds it exactly too.
template <bool INT8, bool VALUES>
__global__ __launch_bounds__(256) void k_quant_rows(const uint16_t* __restrict__ x, int m, uint16_t* __restrict__ xq,
                                                    uint8_t* __restrict__ xc, float* __restrict__ xs) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const uint4* row = reinterpret_cast<const uint4*>(x + (size_t)t * m);
  const int n8 = m / 8;
  float amax = 0.0f;
  for (int i = tid; i < n8; i += 256) {
    const uint4 v = row[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(w[j] & 0xFFFFu))));
      amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(w[j] >> 16))));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int X = act_scale_exponent<INT8>(amax);
  if (tid == 0) xs[t] = ldexpf(1.0f, X);
  for (int i = tid; i < n8; i += 256) {
    const uint4 v = row[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4], c8[2];
    quant8<INT8, VALUES>(w, X, o, c8);
    if (VALUES) reinterpret_cast<uint4*>(xq + (size_t)t * m)[i] = make_uint4(o[0], o[1], o[2], o[3]);
    if (xc) reinterpret_cast<uint2*>(xc + (size_t)t * m)[i] = make_uint2(c8[0], c8[1]);
  }
}

hipError_t launch_quant_rows(const uint16_t* x, int T, int m, bool int8, uint16_t* xq, uint8_t* xc, float* xs,
                             hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (m % 64) return hipErrorInvalidValue;
  const dim3 g((unsigned)T);
  if (int8 && xq)
    k_quant_rows<true, true><<<g, 256, 0, s>>>(x, m, xq, xc, xs);
  else if (int8)
    k_quant_rows<true, false><<<g, 256, 0, s>>>(x, m, xq, xc, xs);
  else if (xq)
    k_quant_rows<false, true><<<g, 256, 0, s>>>(x, m, xq, xc, xs);
  else
    k_quant_rows<false, false><<<g, 256, 0, s>>>(x, m, xq, xc, xs);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s) {
  k_fill_zero<<<grid_for(n / 4 + 1, 8192u), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* src, uint16_t* dst, size_t n, hipStream_t s) {
  k_f32_to_bf16<<<grid_for(n / 4 + 1, 8192u), 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

}  // namespace moe
