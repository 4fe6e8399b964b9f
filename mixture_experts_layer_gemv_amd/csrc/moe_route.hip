// Router product + softmax + top-k, and the expert dispatch (histogram,
// prefix sum, stable permutation), for gfx950 (wave64).
//
// The router maps each token to its experts (HARMOEny article,
// yejing.asia/?p=12, section 3.3 step one; the gating network runs on the GPU
// per the GPU-cache article, coreui.cn, section 3.1).  Dispatch is the
// one-GPU form of sending tokens to their experts (HARMOEny article, section
// 3.3 step four): the assignments are grouped by expert so each expert reads
// a contiguous run of rows.
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

// Single workgroup: counts by LDS atomics, a sequential exclusive scan over
// E <= 64, then a stable scatter chunk by chunk: within a wave, lanes with
// the same expert find each other through six ballots (one per bit of the
// expert id) and rank by lane order; across waves, a per-expert running
// cursor orders the waves.  Assignment order is therefore preserved.
__global__ __launch_bounds__(1024) void k_dispatch(const int32_t* __restrict__ idx, int n, int E,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
  __shared__ int cnt[64];
  __shared__ int offs[65];
  __shared__ int cursor[64];
  __shared__ int wbase[16][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid < 64) {
    cnt[tid] = 0;
    cursor[tid] = 0;
  }
  __syncthreads();
  for (int a = tid; a < n; a += 1024) {
    int e = idx[a];
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      offs[e] = run;
      run += cnt[e];
    }
    offs[E] = run;
  }
  __syncthreads();
  if (tid < E) counts[tid] = cnt[tid];
  if (tid <= E) offsets[tid] = offs[tid];

  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int base = 0; base < n; base += 1024) {
    const int a = base + tid;
    const bool valid = a < n;
    int e = 0;
    if (valid) {
      e = idx[a];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    }
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 6; ++b) {
      const uint64_t mb = __ballot((e >> b) & 1);
      peers &= ((e >> b) & 1) ? mb : ~mb;
    }
    const int rank = __popcll(peers & lt);
    wbase[wave][lane] = 0;
    __syncthreads();
    if (valid && rank == 0) wbase[wave][e] = __popcll(peers);
    __syncthreads();
    if (tid < E) {
      int run = cursor[tid];
      for (int w = 0; w < 16; ++w) {
        const int c = wbase[w][tid];
        wbase[w][tid] = run;
        run += c;
      }
      cursor[tid] = run;
    }
    __syncthreads();
    if (valid) {
      const int pos = offs[e] + wbase[wave][e] + rank;
      perm[pos] = a;
      inv_perm[a] = pos;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_route_topk(const void* x, bool x_bf16, const float* wg, const float* bias, int T, int m, int E,
                             int k, bool logits_in, float* logits, int32_t* idx, float* w, hipStream_t s) {
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
  k_dispatch<<<1, 1024, 0, s>>>(idx, n, E, counts, offsets, perm, inv_perm);
  return hipGetLastError();
}

}  // namespace moe
