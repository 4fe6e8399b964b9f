// Router product + softmax + top-k, and the expert dispatch (histogram,
// prefix sum, stable permutation), for gfx950 (wave64).
//
// The router maps each token to its experts (HARMOEny article,
// yejing.asia/?p=12, section 3.3 step one; the gating network runs on the GPU
// per the GPU-cache article, coreui.cn, section 3.1).  Dispatch is the
// one-GPU form of sending tokens to their experts (HARMOEny article, section
// 3.3 step four): the assignments are grouped by expert so each expert reads
// a contiguous run of rows.
#include "moe_convert.hpp"
#include "moe_dispatch_block.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

// Total order used for ranking: larger value first, NaN below everything,
// +0 == -0.  Returns an unsigned key that compares like the ranking.
__device__ __forceinline__ uint32_t rank_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0u;  // NaN: lowest
  if (u == 0x80000000u) u = 0u;                                          // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float rank_key_value(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;  // key 0 decodes to a NaN
  return __uint_as_float(u);
}

// One step of a recursive-halving reduce-scatter across the wave: each lane
// holds 2H partial sums; afterwards it holds H sums, the half whose index bit
// H matches its own lane bit H.
template <int H>
__device__ __forceinline__ void halve(float* v, int lane) {
  const bool upper = (lane & H) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float send = upper ? v[i] : v[i + H];
    const float keep = upper ? v[i + H] : v[i];
    v[i] = keep + __shfl_xor(send, H, 64);
  }
}

// One wave handles TPW tokens; lane l ends up owning the logit of token
// t0 + l / EB and expert l % EB.  EB * TPW == 64.
template <int EB, int TPW>
__global__ __launch_bounds__(256) void k_route_topk(const void* __restrict__ x, int x_bf16,
                                                     const float* __restrict__ wg, const float* __restrict__ bias,
                                                     int T, int m, int E, int k, int logits_in,
                                                     float* __restrict__ logits, int32_t* __restrict__ idx,
                                                     float* __restrict__ wout) {
  static_assert(EB * TPW == 64, "one logit per lane");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = (blockIdx.x * 4 + wave) * TPW;
  if (t0 >= T) return;
  const int my_t = t0 + lane / EB;
  const int my_e = lane % EB;
  const bool live = my_t < T && my_e < E;

  float v;
  if (logits_in) {
    v = live ? logits[(size_t)my_t * E + my_e] : 0.0f;
  } else {
    float acc[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) acc[i] = 0.0f;
    // lane-strided 8-element chunks of the hidden dimension
    for (int i0 = lane * 8; i0 < m; i0 += 512) {
      float xv[TPW][8];
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        const int t = t0 + tt;
        if (t < T) {
          if (x_bf16) {
            const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + (size_t)t * m + i0);
            const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              xv[tt][2 * j] = __uint_as_float(d[j] << 16);
              xv[tt][2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
            }
          } else {
            const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + (size_t)t * m + i0);
            const float4 a = p[0], b = p[1];
            xv[tt][0] = a.x; xv[tt][1] = a.y; xv[tt][2] = a.z; xv[tt][3] = a.w;
            xv[tt][4] = b.x; xv[tt][5] = b.y; xv[tt][6] = b.z; xv[tt][7] = b.w;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) xv[tt][j] = 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float* row = wg + (size_t)(i0 + j) * E;
#pragma unroll
        for (int e = 0; e < EB; ++e) {
          if (e < E) {
            const float w = row[e];
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) acc[tt * EB + e] = fmaf(xv[tt][j], w, acc[tt * EB + e]);
          }
        }
      }
    }
    halve<32>(acc, lane);
    halve<16>(acc, lane);
    halve<8>(acc, lane);
    halve<4>(acc, lane);
    halve<2>(acc, lane);
    halve<1>(acc, lane);
    v = acc[0];
    if (live && bias) v += bias[my_e];
    if (live && logits) logits[(size_t)my_t * E + my_e] = v;
  }

  // top-k inside each aligned group of EB lanes (one token per group):
  // key = (rank of the logit, then lower expert index first)
  uint64_t key = live ? (((uint64_t)rank_key(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)my_e)) : 0ull;
  uint64_t mine = 0ull;  // the winner of round j, kept by the group's lane j
  float l0 = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key;
#pragma unroll
    for (int off = 1; off < EB; off <<= 1) {
      const uint64_t o = __shfl_xor(best, off, 64);
      best = o > best ? o : best;
    }
    if (j == 0) l0 = rank_key_value((uint32_t)(best >> 32));
    if (my_e == j) mine = best;
    if (key == best) key = 0ull;
  }
  // gate weights: softmax over the selected k (slot order)
  const bool slot = live && my_e < k;
  const float lj = rank_key_value((uint32_t)(mine >> 32));
  float ex = slot ? expf(lj - l0) : 0.0f;
  float den = ex;
#pragma unroll
  for (int off = 1; off < EB; off <<= 1) den += __shfl_xor(den, off, 64);
  if (slot) {
    idx[(size_t)my_t * k + my_e] = (int32_t)(0xFFFFFFFFu - (uint32_t)(mine & 0xFFFFFFFFull));
    wout[(size_t)my_t * k + my_e] = ex / den;
  }
}

// Top-k of one token held one logit per lane (lanes >= E hold nothing):
// k rounds of a wave-wide max over 64-bit keys (rank of the logit, then the
// lower expert index), then the softmax over the selected logits.  Lane j < k
// writes slot j.
__device__ __forceinline__ void wave_topk_write(float v, bool live, int e, int k, int32_t* idx_row,
                                                float* w_row) {
  uint64_t key = live ? (((uint64_t)rank_key(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e)) : 0ull;
  uint64_t mine = 0ull;
  float l0 = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint64_t o = __shfl_xor(best, off, 64);
      best = o > best ? o : best;
    }
    if (j == 0) l0 = rank_key_value((uint32_t)(best >> 32));
    if (e == j) mine = best;
    if (key == best) key = 0ull;
  }
  const bool slot = e < k;
  const float lj = rank_key_value((uint32_t)(mine >> 32));
  const float ex = slot ? expf(lj - l0) : 0.0f;
  float den = ex;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) den += __shfl_xor(den, off, 64);
  if (slot) {
    idx_row[e] = (int32_t)(0xFFFFFFFFu - (uint32_t)(mine & 0xFFFFFFFFull));
    w_row[e] = ex / den;
  }
}

// Recursive-halving step over lane bit B on an array of N partial sums: the
// lane keeps the half selected by its bit B and adds the partner's copy.
template <int B, int N>
__device__ __forceinline__ void halve_bit(float* v, int lane) {
  const bool upper = (lane >> B) & 1;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float send = upper ? v[i] : v[i + N / 2];
    const float keep = upper ? v[i + N / 2] : v[i];
    v[i] = keep + __shfl_xor(send, 1 << B, 64);
  }
}

template <int E, int TB>
struct RouteShape {
  static constexpr int Q = E / 4;                                  // lanes per router-weight row (16 B each)
  static constexpr int LQ = E == 8 ? 1 : E == 16 ? 2 : E == 32 ? 3 : 4;
  static constexpr int RPC = 64 / Q;                               // rows per 1 KiB chunk
  static constexpr int NV = TB * 4;                                // partial sums per lane
  static constexpr int STEPS = 6 - LQ;                             // lane bits that index rows
  static constexpr bool HALVING = NV >= (1 << STEPS);              // enough sums for a reduce-scatter
  static constexpr int PER = HALVING ? (NV >> STEPS) : NV;         // sums a lane holds afterwards
};

template <int B, int LQ, int N>
__device__ __forceinline__ void halve_down(float* v, int lane) {
  if constexpr (B >= LQ) {
    halve_bit<B, N>(v, lane);
    halve_down<B - 1, LQ, N / 2>(v, lane);
  }
}

template <int LQ, int N>
__device__ __forceinline__ void butterfly_rows(float* v) {
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int b = LQ; b < 6; ++b) v[i] += __shfl_xor(v[i], 1 << b, 64);
}

constexpr int kRouteLdsX = 128 * 1024;  // most bytes of staged activations per block

// Bytes of activations a block of TB tokens can stage; the host checks
// TB * m * sizeof(x) against the same figure.
constexpr int route_lds_bytes(int tb) { return tb * 65536 < kRouteLdsX ? tb * 65536 : kRouteLdsX; }

// Router for E in {8, 16, 32, 64}: one block of NW waves per TB tokens
// (TB * E <= 128, NW >= TB), staging at most LX bytes of activation rows.
// 16 waves and up to 128 KiB by default; large batches of rows of at most
// 8 KiB take 8 tokens on 8 waves in 64 KiB, so that two blocks share a CU
// and one stages its rows while the other multiplies.  The tokens'
// activation rows are staged in LDS; each wave streams 1 KiB chunks of the
// router weights with one coalesced 16-byte load per lane (lane =
// row-in-chunk x expert quad) and keeps TB x 4 partial sums.
// Sums over rows: across the lanes of a wave (reduce-scatter when there are
// enough partials, butterfly otherwise), then a fixed-order sum over the NW
// waves in LDS.  One wave per token then takes the top-k.  The block also
// zeroes its tokens' rows of the fp32 output accumulator.
__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Residual element i as fp32.
__device__ __forceinline__ float residual_at(const RouteFuse& F, size_t i) {
  return F.res_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(F.residual)[i])
                    : static_cast<const float*>(F.residual)[i];
}

template <int E, int TB, bool XBF16, int NW = 16, int LX = route_lds_bytes(TB)>
__global__ __launch_bounds__(64 * NW) void k_route_fast(const void* __restrict__ x, const float* __restrict__ wg,
                                                     const float* __restrict__ bias, int T, int m, int k,
                                                     float* __restrict__ logits, int32_t* __restrict__ idx,
                                                     float* __restrict__ wout, float* __restrict__ yacc, int ym,
                                                     const RouteFuse F) {
  using S = RouteShape<E, TB>;
  static_assert(TB * E <= 128 && TB <= 16 && NW >= TB && NW <= 16, "block shape");
  constexpr int XB = XBF16 ? 2 : 4;
  constexpr int NT = 64 * NW;  // threads
  __shared__ __attribute__((aligned(16))) unsigned char xs_raw[LX];
  __shared__ float red[NW][TB * E];
  __shared__ float lg[TB][E];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * TB;
  const int nt = min(TB, T - t0);

  if (yacc && F.residual) {
    const size_t base = (size_t)t0 * ym;
    for (int i = tid; i < nt * ym; i += NT) yacc[base + i] = residual_at(F, base + i);
  } else if (yacc) {
    float4* yr = reinterpret_cast<float4*>(yacc + (size_t)t0 * ym);
    const int n4 = nt * ym / 4;
    for (int i = tid; i < n4; i += NT) yr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // The router weights: the wave's chunks are c = wave, wave + NW, ...; each
  // group of WU of them is loaded whole (a chunk past the end reloads the
  // group's first) while the group before it is multiplied, and the first
  // group while the rows are staged.
  const int q = lane & (S::Q - 1);
  const int rr = lane >> S::LQ;
  const int nchunks = m / S::RPC;
  constexpr int WU = 8;
  auto load_group = [&](int c0, float4(&wv)[WU]) {
#pragma unroll
    for (int u = 0; u < WU; ++u) {
      const int c = c0 + NW * u < nchunks ? c0 + NW * u : c0;
      wv[u] = *reinterpret_cast<const float4*>(wg + (size_t)(c * S::RPC + rr) * E + 4 * q);
    }
  };
  float4 wv[WU];
  if (wave < nchunks) load_group(wave, wv);

  // stage x rows [t0, t0 + nt) (rows past T are zero), eight loads in flight
  // per thread before the first LDS write
  {
    const int row16 = m * XB / 16, n16 = TB * row16, live16 = nt * row16;
    uint4* dst = reinterpret_cast<uint4*>(xs_raw);
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(x) + (size_t)t0 * m * XB);
    constexpr int U = 8;
    for (int i0 = tid; i0 < n16; i0 += NT * U) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + NT * u;
        v[u] = i < live16 ? src[i] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + NT * u;
        if (i < n16) dst[i] = v[u];
      }
    }
  }
  __syncthreads();
  if (F.norm) {
    // Norm of the staged rows (the reductions along the row inside this
    // block, one wave per token), in place, so the router and the experts
    // both see the normalised rows; they also go to F.xn for the experts.
    // Rows are read and written 16 bytes at a time (EV elements; m is a
    // multiple of 64), gamma and beta likewise.
    __shared__ float mu_s[TB], r_s[TB];
    constexpr int EV = XBF16 ? 8 : 4;
    const int mv = m / EV;  // 16-byte vectors per row
    uint4* const xv4 = reinterpret_cast<uint4*>(xs_raw);
    auto unpack = [](const uint4& v, float (&f)[EV]) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (XBF16) {
          f[2 * j] = __uint_as_float(w[j] << 16);
          f[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        } else {
          f[j] = __uint_as_float(w[j]);
        }
      }
    };
    if (wave < nt) {
      float mu = 0.0f;
      if (F.norm == 1) {
        float sum = 0.0f;
        for (int i = lane; i < mv; i += 64) {
          float f[EV];
          unpack(xv4[wave * mv + i], f);
#pragma unroll
          for (int j = 0; j < EV; ++j) sum += f[j];
        }
        mu = wave_sum64(sum) / (float)m;
      }
      float ss = 0.0f;
      for (int i = lane; i < mv; i += 64) {
        float f[EV];
        unpack(xv4[wave * mv + i], f);
#pragma unroll
        for (int j = 0; j < EV; ++j) {
          const float d = f[j] - mu;
          ss = fmaf(d, d, ss);
        }
      }
      ss = wave_sum64(ss);
      if (lane == 0) {
        mu_s[wave] = mu;
        r_s[wave] = 1.0f / sqrtf(ss / (float)m + F.eps);
      }
    }
    __syncthreads();
    uint4* const xn4 = reinterpret_cast<uint4*>(static_cast<char*>(F.xn) + (size_t)t0 * m * XB);
    const bool with_beta = F.norm == 1 && F.beta;
    for (int i = tid; i < nt * mv; i += NT) {
      const int t = i / mv, c0 = (i - t * mv) * EV;
      float f[EV], g[EV], b[EV];
      unpack(xv4[i], f);
#pragma unroll
      for (int j = 0; j < EV; j += 4) {
        const float4 g4 = *reinterpret_cast<const float4*>(F.gamma + c0 + j);
        g[j] = g4.x, g[j + 1] = g4.y, g[j + 2] = g4.z, g[j + 3] = g4.w;
        const float4 b4 = with_beta ? *reinterpret_cast<const float4*>(F.beta + c0 + j) : make_float4(0.f, 0.f, 0.f, 0.f);
        b[j] = b4.x, b[j + 1] = b4.y, b[j + 2] = b4.z, b[j + 3] = b4.w;
      }
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < EV; ++j) {
        float v = (f[j] - mu_s[t]) * r_s[t] * g[j];
        if (with_beta) v += b[j];
        if constexpr (XBF16) {
          const uint32_t h = f32_to_bf16(v);
          if (j & 1)
            w[j >> 1] |= h << 16;
          else
            w[j >> 1] = h;
        } else {
          w[j] = __float_as_uint(v);
        }
      }
      const uint4 o = make_uint4(w[0], w[1], w[2], w[3]);
      xv4[i] = o;
      xn4[i] = o;
    }
    __syncthreads();
  }

  if constexpr (XBF16) {
    if (F.quant) {
      // 8-bit activations: each staged row's scale (wave t reduces row t),
      // then the rows' codes and values, eight elements per 16-byte LDS read
      __shared__ int qx_s[TB];
      const int m8 = m / 8;
      const uint4* x8 = reinterpret_cast<const uint4*>(xs_raw);
      const bool int8 = F.quant == 2;
      if (wave < nt) {
        float amax = 0.0f;
        for (int c = lane; c < m8; c += 64) {
          const uint4 v = x8[wave * m8 + c];
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[j] << 16)), fabsf(__uint_as_float(w[j] & 0xFFFF0000u))));
        }
        amax = wave_max64(amax);
        const int X = int8 ? act_scale_exponent<true>(amax) : act_scale_exponent<false>(amax);
        if (lane == 0) {
          qx_s[wave] = X;
          F.xs[t0 + wave] = ldexpf(1.0f, X);
        }
      }
      __syncthreads();
      uint4* q8 = F.xq ? reinterpret_cast<uint4*>(F.xq + (size_t)t0 * m) : nullptr;
      uint2* c8 = F.xc ? reinterpret_cast<uint2*>(F.xc + (size_t)t0 * m) : nullptr;
      for (int i = tid; i < nt * m8; i += NT) {
        const uint4 v = x8[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        const int X = qx_s[i / m8];
        uint32_t o[4], c[2];
        if (int8) {
          if (q8) quant8<true, true>(w, X, o, c); else quant8<true, false>(w, X, o, c);
        } else {
          if (q8) quant8<false, true>(w, X, o, c); else quant8<false, false>(w, X, o, c);
        }
        if (q8) q8[i] = make_uint4(o[0], o[1], o[2], o[3]);
        if (c8) c8[i] = make_uint2(c[0], c[1]);
      }
    }
  }

  float acc[S::NV];
#pragma unroll
  for (int i = 0; i < S::NV; ++i) acc[i] = 0.0f;
  // the products keep increasing c
  for (int c0 = wave; c0 < nchunks; c0 += NW * WU) {
    float4 wn[WU];
    const bool more = c0 + NW * WU < nchunks;
    if (more) load_group(c0 + NW * WU, wn);
#pragma unroll
    for (int u = 0; u < WU; ++u) {
      const int c = c0 + NW * u;
      if (c < nchunks) {
        const int r = c * S::RPC + rr;
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          float xv;
          if constexpr (XBF16)
            xv = bf16_to_f32(reinterpret_cast<const uint16_t*>(xs_raw)[t * m + r]);
          else
            xv = reinterpret_cast<const float*>(xs_raw)[t * m + r];
          acc[t * 4 + 0] = fmaf(xv, wv[u].x, acc[t * 4 + 0]);
          acc[t * 4 + 1] = fmaf(xv, wv[u].y, acc[t * 4 + 1]);
          acc[t * 4 + 2] = fmaf(xv, wv[u].z, acc[t * 4 + 2]);
          acc[t * 4 + 3] = fmaf(xv, wv[u].w, acc[t * 4 + 3]);
        }
      }
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < WU; ++u) wv[u] = wn[u];
    }
  }
  // sum over the row lanes (lane bits LQ..5)
  if constexpr (S::HALVING) {
    halve_down<5, S::LQ, S::NV>(acc, lane);
    const int L = lane >> S::LQ;
#pragma unroll
    for (int i = 0; i < S::PER; ++i) {
      const int v = L * S::PER + i;  // partial index t*4 + j
      red[wave][(v >> 2) * E + 4 * q + (v & 3)] = acc[i];
    }
  } else {
    butterfly_rows<S::LQ, S::NV>(acc);
    if (rr == 0) {
#pragma unroll
      for (int v = 0; v < S::NV; ++v) red[wave][(v >> 2) * E + 4 * q + (v & 3)] = acc[v];
    }
  }
  __syncthreads();
  if (tid < TB * E) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[w][tid];
    const int t = tid / E, e = tid % E;
    if (bias) s += bias[e];
    lg[t][e] = s;
    if (logits && t < nt) logits[(size_t)(t0 + t) * E + e] = s;
  }
  __syncthreads();
  if (wave < nt) {
    const int t = t0 + wave;
    const bool live = lane < E;
    wave_topk_write(live ? lg[wave][lane] : 0.0f, live, lane, k, idx + (size_t)t * k, wout + (size_t)t * k);
  }
}

// The dispatch over workgroups of 16 waves, workgroup b placing assignments
// [b * chunk, (b + 1) * chunk).  Every workgroup counts all n expert ids
// itself, so no workgroup waits for another: a wave finds the lanes holding
// the same expert with six ballots (as in the ranking) and the lowest of them
// adds the group's size to the wave's own LDS row of counts, once for every
// id and once for the ids before the workgroup's range.  The sums over the
// waves give the experts' counts (hence offsets) and each expert's
// assignments ahead of the range; the range is then ranked as in the one-
// workgroup dispatch, its cursors starting there.  Workgroup 0 publishes
// counts and offsets.
__global__ __launch_bounds__(1024) void k_dispatch(const int32_t* __restrict__ idx, int n, int E, int chunk,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
  constexpr int NW = 16, U = 4;
  __shared__ DispatchLds<NW> L;
  __shared__ int wtot[NW][64], wpre[NW][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lo = blockIdx.x * chunk, hi = min(n, lo + chunk);
  wtot[wave][lane] = 0;
  wpre[wave][lane] = 0;
  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (long long base = 0; base < n; base += NW * 64 * U) {  // 64-bit: n may be near 2^31
    int ev[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long a = base + u * NW * 64 + tid;
      ev[u] = a < n ? idx[a] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long a = base + u * NW * 64 + tid;
      const bool valid = a < n;
      const int e = valid ? clamp_expert(ev[u], E) : 0;
      uint64_t peers = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 6; ++b) {
        const uint64_t mb = __ballot((e >> b) & 1);
        peers &= ((e >> b) & 1) ? mb : ~mb;
      }
      const uint64_t before = __ballot(a < lo);
      if (valid && __popcll(peers & lt) == 0) {  // the group's lowest lane; distinct experts per wave
        wtot[wave][e] += __popcll(peers);
        wpre[wave][e] += __popcll(peers & before);
      }
    }
  }
  __syncthreads();
  if (tid < 64) {
    int tot = 0, pre = 0;
    for (int w = 0; w < NW; ++w) {
      tot += wtot[w][tid];
      pre += wpre[w][tid];
    }
    L.cnt[tid] = tot;
    L.cursor[tid] = pre;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      L.offs[e] = run;
      run += L.cnt[e];
    }
    L.offs[E] = run;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < E) counts[tid] = L.cnt[tid];
    if (tid <= E) offsets[tid] = L.offs[tid];
  }
  block_stable_positions_range<NW>(idx, lo, hi, E, L, [&](int a, int, int pos) {
    perm[pos] = a;
    inv_perm[a] = pos;
  });
}

// One block per row: the row's norm written to F.xn (the unfused form).
template <bool XBF16>
__global__ __launch_bounds__(256) void k_norm_rows(const void* __restrict__ x, int m, const RouteFuse F) {
  // 16 bytes (EV elements) of the row per thread and step; m is a multiple
  // of 64, gamma, beta and the rows 16-byte aligned
  constexpr int EV = XBF16 ? 8 : 4;
  __shared__ float part[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mv = m / EV;
  const uint4* const row = reinterpret_cast<const uint4*>(static_cast<const char*>(x) + (size_t)t * m * (XBF16 ? 2 : 4));
  uint4* const out = reinterpret_cast<uint4*>(static_cast<char*>(F.xn) + (size_t)t * m * (XBF16 ? 2 : 4));
  auto unpack = [](const uint4& v, float (&f)[EV]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (XBF16) {
        f[2 * j] = __uint_as_float(w[j] << 16);
        f[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      } else {
        f[j] = __uint_as_float(w[j]);
      }
    }
  };
  auto block_sum = [&](float v) {
    v = wave_sum64(v);
    if (lane == 0) part[wave] = v;
    __syncthreads();
    const float r = part[0] + part[1] + part[2] + part[3];
    __syncthreads();
    return r;
  };
  float mu = 0.0f;
  if (F.norm == 1) {
    float sum = 0.0f;
    for (int i = tid; i < mv; i += 256) {
      float f[EV];
      unpack(row[i], f);
#pragma unroll
      for (int j = 0; j < EV; ++j) sum += f[j];
    }
    mu = block_sum(sum) / (float)m;
  }
  float ss = 0.0f;
  for (int i = tid; i < mv; i += 256) {
    float f[EV];
    unpack(row[i], f);
#pragma unroll
    for (int j = 0; j < EV; ++j) {
      const float d = f[j] - mu;
      ss = fmaf(d, d, ss);
    }
  }
  const float r = 1.0f / sqrtf(block_sum(ss) / (float)m + F.eps);
  const bool with_beta = F.norm == 1 && F.beta;
  for (int i = tid; i < mv; i += 256) {
    const int c0 = i * EV;
    float f[EV];
    unpack(row[i], f);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < EV; j += 4) {
      const float4 g4 = *reinterpret_cast<const float4*>(F.gamma + c0 + j);
      const float4 b4 = with_beta ? *reinterpret_cast<const float4*>(F.beta + c0 + j) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float g[4] = {g4.x, g4.y, g4.z, g4.w}, bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v = (f[j + q] - mu) * r * g[q];
        if (with_beta) v += bb[q];
        if constexpr (XBF16) {
          const uint32_t h = f32_to_bf16(v);
          if ((j + q) & 1)
            w[(j + q) >> 1] |= h << 16;
          else
            w[(j + q) >> 1] = h;
        } else {
          w[j + q] = __float_as_uint(v);
        }
      }
    }
    out[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__global__ __launch_bounds__(256) void k_fill_residual(float* __restrict__ yacc, size_t n, const RouteFuse F) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) yacc[i] = residual_at(F, i);
}

}  // namespace

hipError_t launch_route_topk(const void* x, bool x_bf16, const float* wg, const float* bias, int T, int m, int E,
                             int k, bool logits_in, float* logits, int32_t* idx, float* w, float* yacc, int ym,
                             hipStream_t s, const RouteFuse* fuse) {
  const int xb = x_bf16 ? 2 : 4;
  const RouteFuse F = fuse ? *fuse : RouteFuse{};
  if (F.norm && (logits_in || !F.gamma || !F.xn)) return hipErrorInvalidValue;
  if (F.quant && (logits_in || !x_bf16 || !F.xs || (!F.xq && !F.xc) || m % 64)) return hipErrorInvalidValue;
  if (T <= 0) return hipSuccess;
  if (!logits_in && (E == 8 || E == 16 || E == 32 || E == 64) && (yacc == nullptr || ym % 4 == 0)) {
    // tokens per block: one up to 256 tokens (spreads the router weights'
    // reads over T CUs; at 256 tokens of 4096 and 16 experts, 9.8 against
    // 12.7 us for four), up to 128 / E for large batches
    const int tb_max = 128 / E < 16 ? 128 / E : 16;
    // past 1024 tokens, eight tokens per 512-thread block with 64 KiB of
    // staged rows (two blocks per CU) where they fit
    if (T > 1024 && tb_max >= 8 && 8 * m * xb <= 65536) {
      const unsigned grid = (unsigned)((T + 7) / 8);
#define MOE_ROUTE_HALF(EE)                                                                                    \
  if (E == EE) {                                                                                              \
    if (x_bf16)                                                                                               \
      k_route_fast<EE, 8, true, 8, 65536><<<grid, 512, 0, s>>>(x, wg, bias, T, m, k, logits, idx, w, yacc, ym, F); \
    else                                                                                                      \
      k_route_fast<EE, 8, false, 8, 65536><<<grid, 512, 0, s>>>(x, wg, bias, T, m, k, logits, idx, w, yacc, ym, F); \
    return hipGetLastError();                                                                                 \
  }
      MOE_ROUTE_HALF(8)
      MOE_ROUTE_HALF(16)
#undef MOE_ROUTE_HALF
    }
    const int tb = T <= 256 ? 1 : (T <= 1024 ? (4 < tb_max ? 4 : tb_max) : tb_max);
    if (tb * m * xb <= route_lds_bytes(tb)) {
      const unsigned grid = (unsigned)((T + tb - 1) / tb);
#define MOE_ROUTE_FAST(EE, TT)                                                                               \
  if (E == EE && tb == TT) {                                                                                 \
    if (x_bf16)                                                                                              \
      k_route_fast<EE, TT, true><<<grid, 1024, 0, s>>>(x, wg, bias, T, m, k, logits, idx, w, yacc, ym, F);   \
    else                                                                                                     \
      k_route_fast<EE, TT, false><<<grid, 1024, 0, s>>>(x, wg, bias, T, m, k, logits, idx, w, yacc, ym, F);  \
    return hipGetLastError();                                                                                \
  }
      MOE_ROUTE_FAST(8, 1)
      MOE_ROUTE_FAST(8, 4)
      MOE_ROUTE_FAST(16, 1)
      MOE_ROUTE_FAST(16, 4)
      MOE_ROUTE_FAST(16, 8)
      MOE_ROUTE_FAST(32, 1)
      MOE_ROUTE_FAST(32, 4)
      MOE_ROUTE_FAST(64, 1)
      MOE_ROUTE_FAST(64, 2)
#undef MOE_ROUTE_FAST
    }
  }
  if (F.norm) {  // unfused: the rows' norm first, then the router on them
    if (x_bf16)
      k_norm_rows<true><<<T, 256, 0, s>>>(x, m, F);
    else
      k_norm_rows<false><<<T, 256, 0, s>>>(x, m, F);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    x = F.xn;
  }
  if (yacc && F.residual) {
    k_fill_residual<<<(unsigned)(((size_t)T * ym + 255) / 256), 256, 0, s>>>(yacc, (size_t)T * ym, F);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (yacc) {
    const hipError_t e = launch_fill_zero(yacc, (size_t)T * ym, s);
    if (e != hipSuccess) return e;
  }
  if (F.quant) {  // the experts' rows: x, or the normalised rows written above
    const hipError_t e = launch_quant_rows(static_cast<const uint16_t*>(x), T, m, F.quant == 2, F.xq, F.xc, F.xs, s);
    if (e != hipSuccess) return e;
  }
  if (E <= 8) {
    const int tpb = 4 * 8;
    k_route_topk<8, 8><<<(T + tpb - 1) / tpb, 256, 0, s>>>(x, x_bf16, wg, bias, T, m, E, k, logits_in, logits,
                                                            idx, w);
  } else if (E <= 16) {
    const int tpb = 4 * 4;
    k_route_topk<16, 4><<<(T + tpb - 1) / tpb, 256, 0, s>>>(x, x_bf16, wg, bias, T, m, E, k, logits_in, logits,
                                                             idx, w);
  } else if (E <= 32) {
    const int tpb = 4 * 2;
    k_route_topk<32, 2><<<(T + tpb - 1) / tpb, 256, 0, s>>>(x, x_bf16, wg, bias, T, m, E, k, logits_in, logits,
                                                             idx, w);
  } else {
    const int tpb = 4;
    k_route_topk<64, 1><<<(T + tpb - 1) / tpb, 256, 0, s>>>(x, x_bf16, wg, bias, T, m, E, k, logits_in, logits,
                                                             idx, w);
  }
  return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* idx, int n, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv_perm, hipStream_t s) {
  if (n < 0 || E < 1 || E > 64) return hipErrorInvalidValue;
  // ranges of whole 1024-assignment passes, at most 64 workgroups (each one
  // reads all n ids to count them)
  const int passes = (n + 1023) / 1024;
  const int chunk = 1024 * ((passes + 63) / 64 > 1 ? (passes + 63) / 64 : 1);
  const int grid = n > 0 ? (n + chunk - 1) / chunk : 1;
  k_dispatch<<<grid, 1024, 0, s>>>(idx, n, E, chunk, counts, offsets, perm, inv_perm);
  return hipGetLastError();
}

}  // namespace moe
