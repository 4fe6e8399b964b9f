// Expert FFN for decode-sized batches: a skinny grouped GEMM that streams each
// touched expert's weights from HBM once and multiplies them by that expert's
// few activation rows on the matrix cores.
//
// Design (prior art: the small-batch GEMM of the DeepSpeed-Inference summary,
// datalearner.com, section 3 "SBI-GeMM"):
//  - tiling along the output dimension: a workgroup owns a 16-column tile of
//    one expert (both SwiGLU streams of it), so the reduction stays inside the
//    workgroup (part 1 of that section).  When outputs are too few to keep
//    every CU streaming, the reduction dimension is also split over
//    workgroups (its two-kernel variant); here the split partials meet in the
//    fp32 atomic combine, so no second kernel is needed;
//  - inside the workgroup the reduction dimension is split over the waves and
//    the partial tiles are summed through one LDS transpose, after which each
//    thread reads its outputs' partials contiguously (part 2, with wave64);
//  - weights are re-laid out at initialisation so a wave's load is 1 KiB of
//    contiguous memory (part 3; see the packed layout in moe_kernels.hpp);
//  - small-batch work is bandwidth-bound, so the activations (a few rows per
//    expert) ride along in registers and the product runs on MFMA.
// Work items are (column tile, reduction slice, expert, row chunk) tuples
// generated on the device from the dispatch offsets: the host never reads the
// expert counts.  With `topk_idx` set, each workgroup derives the dispatch
// itself in its prologue (and logical workgroup 0 publishes it), so no
// separate dispatch launch is needed.
#include "moe_dispatch_block.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// 8 signed bytes (two dwords) -> 8 bf16.  |q| <= 128 is exact in bf16, so the
// fp32 value's upper half is the bf16 pattern.
__device__ __forceinline__ bf16x8_t i8x8_to_bf16(uint32_t lo, uint32_t hi) {
  u32x4_t r;
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
  return as_bf16x8(r);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

template <int MT, int G, bool I8, int EPI, int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(MT * (I8 ? 2 : 1) >= 4 ? 2 : 4))) void
k_ffn_skinny(const SkinnyArgs A) {
  constexpr int NT = NW * 64;
  constexpr int R = 16 * MT;        // rows per work item
  constexpr int AH = I8 ? 2 : 1;    // activation loads per K unit
  constexpr int UK = I8 ? 64 : 32;  // k per unit
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  __shared__ DispatchLds<NW> DL;
  __shared__ int offs_s[kMaxExperts + 1];
  __shared__ int rows_s[R];
  __shared__ float red[NW * G * MT * 256];

  // Block -> logical work index: consecutive logical indices stay on one XCD
  // (blocks are dealt to the 8 XCDs round-robin), so the row chunks of one
  // (expert, tile) run together and share that XCD's L2 copy of the weights.
  const int nblk = gridDim.x;  // multiple of 8
  const int b = blockIdx.x;
  const int L = (b & 7) * (nblk >> 3) + (b >> 3);
  const int NB = A.N / 16;
  const int S = A.ksplit;
  const int ntile = L / (A.W * S);
  const int rem0 = L - ntile * (A.W * S);
  const int ks = rem0 / A.W;
  const int pair = rem0 - ks * A.W;
  const int n_assign = A.T * A.topk;

  if (A.topk_idx) {
    block_histogram<NW>(A.topk_idx, n_assign, A.E, DL);
    if (tid <= A.E) offs_s[tid] = DL.offs[tid];
  } else {
    if (tid <= A.E) offs_s[tid] = A.offsets[tid];
  }
  __syncthreads();

  // (expert, chunk) of this work item and the number of valid pairs
  int e = -1, chunk = 0, npairs = 0;
  for (int i = 0; i < A.E; ++i) {
    const int nch = (offs_s[i + 1] - offs_s[i] + R - 1) / R;
    if (e < 0 && pair < npairs + nch) {
      e = i;
      chunk = pair - npairs;
    }
    npairs += nch;
  }
  const bool valid = ntile < NB && e >= 0;
  const int row0 = valid ? offs_s[e] + chunk * R : 0;
  const int nrows = valid ? min(R, offs_s[e + 1] - row0) : 0;

  if (A.topk_idx) {
    const bool publish = L == 0;
    if (publish || valid) {
      block_stable_positions<NW>(A.topk_idx, n_assign, A.E, DL, [&](int a, int ea, int pos) {
        if (publish) {
          A.d_perm[pos] = a;
          A.d_inv[a] = pos;
        }
        if (valid && ea == e && pos >= row0 && pos < row0 + nrows) rows_s[pos - row0] = a;
      });
      if (publish) {
        if (tid < A.E) A.d_counts[tid] = DL.cnt[tid];
        if (tid <= A.E) A.d_offsets[tid] = DL.offs[tid];
      }
    }
  } else if (valid && A.gather) {
    if (tid < nrows) rows_s[tid] = A.perm[row0 + tid];
    __syncthreads();
  }
  if (!valid) return;

  // Activation row pointers of this lane, one per M tile.  Lanes past the
  // chunk's last row read a valid row (the chunk's first) so every load is
  // unconditional; their output rows are never stored.
  const uint16_t* arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = mt * 16 + (lane & 15);
    const int rr = r < nrows ? r : 0;
    const int src = A.gather ? rows_s[rr] / A.topk : row0 + rr;
    arow[mt] = A.act + (size_t)src * A.K + 8 * (lane >> 4);
  }

  const int U = A.K / UK;
  const int part = ks * NW + wave;
  const int u0 = (int)(((long long)part * U) / (S * NW));
  const int u1 = (int)(((long long)(part + 1) * U) / (S * NW));
  const u32x4_t* wp = static_cast<const u32x4_t*>(A.w) + (size_t)(e * NB + ntile) * U * G * 64 + lane;

  floatx4_t acc[G][MT];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[g][mt] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4_t wb[D][G];
  u32x4_t ab[D][MT][AH];

#define MOE_ISSUE(slot, u)                                                                             \
  do {                                                                                                 \
    _Pragma("unroll") for (int g = 0; g < G; ++g) wb[slot][g] =                                        \
        __builtin_nontemporal_load(wp + ((size_t)(u) * G + g) * 64);                                   \
    _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) _Pragma("unroll") for (int h = 0; h < AH; ++h)   \
        ab[slot][mt][h] = *reinterpret_cast<const u32x4_t*>(arow[mt] + (size_t)(u) * UK + 32 * h);     \
  } while (0)

#define MOE_CONSUME(slot)                                                                              \
  do {                                                                                                 \
    if constexpr (I8) {                                                                                \
      _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                                  \
        _Pragma("unroll") for (int g = 0; g < G; ++g) {                                                \
          const u32x4_t q = wb[slot][g];                                                               \
          const bf16x8_t bw = h == 0 ? i8x8_to_bf16(q[0], q[1]) : i8x8_to_bf16(q[2], q[3]);            \
          _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) acc[g][mt] =                               \
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ab[slot][mt][h]), bw, acc[g][mt], 0, 0, 0); \
        }                                                                                              \
      }                                                                                                \
    } else {                                                                                           \
      _Pragma("unroll") for (int g = 0; g < G; ++g) {                                                  \
        const bf16x8_t bw = as_bf16x8(wb[slot][g]);                                                    \
        _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) acc[g][mt] =                                 \
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ab[slot][mt][0]), bw, acc[g][mt], 0, 0, 0); \
      }                                                                                                \
    }                                                                                                  \
  } while (0)

  // Software pipeline, D units in flight.  When the wave has at least 2D
  // units: an unguarded prologue and steady state (straight-line code, so the
  // compiler waits only for the unit being consumed), then a guarded tail of
  // fewer than 2D units.  Short reductions take a plain loop.
  if (u1 - u0 >= 2 * D) {
#pragma unroll
    for (int d = 0; d < D; ++d) MOE_ISSUE(d, u0 + d);
    int u = u0;
    for (; u + 2 * D <= u1; u += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        MOE_CONSUME(d);
        MOE_ISSUE(d, u + d + D);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (u + d < u1) {
        MOE_CONSUME(d);
        if (u + d + D < u1) MOE_ISSUE(d, u + d + D);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (u + D + d < u1) MOE_CONSUME(d);
  } else {
    for (int u = u0; u < u1; ++u) {
      MOE_ISSUE(0, u);
      MOE_CONSUME(0);
    }
  }
#undef MOE_CONSUME
#undef MOE_ISSUE

  // Cross-wave reduction through one LDS transpose: wave w writes its partial
  // tile; each output's NW partials are then read by one thread.
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[((wave * G + g) * MT + mt) * 256 + i * 64 + lane] = acc[g][mt][i];
  __syncthreads();

  for (int o = tid; o < MT * 256; o += NT) {
    const int mt = o >> 8, i = (o >> 6) & 3, ln = o & 63;
    const int row = mt * 16 + 4 * (ln >> 4) + i;
    if (row >= nrows) continue;
    const int col = ntile * 16 + (ln & 15);
    float v[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red[((w * G + g) * MT + mt) * 256 + i * 64 + ln];
      v[g] = s;
    }
    const int r = row0 + row;
    if constexpr (EPI == EPI_UP_SWIGLU) {
      float gv = v[0], uv = v[G - 1];
      if constexpr (I8) {
        gv *= A.scale0[(size_t)e * A.N + col];
        uv *= A.scale1[(size_t)e * A.N + col];
      }
      A.h_out[(size_t)r * A.N + col] = f32_to_bf16(silu(gv) * uv);
    } else if constexpr (EPI == EPI_UP_RELU) {
      float gv = v[0];
      if constexpr (I8) gv *= A.scale0[(size_t)e * A.N + col];
      A.h_out[(size_t)r * A.N + col] = f32_to_bf16(gv > 0.0f ? gv : 0.0f);
    } else {
      float o2 = v[0];
      if constexpr (I8) o2 *= A.scale0[(size_t)e * A.N + col];
      if constexpr (EPI == EPI_DOWN_ACC) {
        const int a = A.perm[r];
        unsafeAtomicAdd(A.f_out + (size_t)(a / A.topk) * A.N + col, A.topk_w[a] * o2);
      } else {
        A.f_out[(size_t)r * A.N + col] = o2;
      }
    }
  }

}

// Units in flight per wave: enough bytes outstanding per CU to cover HBM
// latency while the register budget keeps several waves per SIMD.
constexpr int depth(int mt, int g, bool i8) { return (mt * (i8 ? 2 : 1) + g) <= 3 ? 6 : 4; }

template <int MT, bool I8>
hipError_t launch_mt(const SkinnyArgs& a, int epi, hipStream_t s) {
  const int NB = a.N / 16;
  const long long work = (long long)NB * a.W * a.ksplit;
  const long long nblk = (work + 7) / 8 * 8;
  const dim3 grid((unsigned)nblk);
  switch (epi) {
    case EPI_UP_SWIGLU:
      k_ffn_skinny<MT, 2, I8, EPI_UP_SWIGLU, depth(MT, 2, I8), 4><<<grid, 256, 0, s>>>(a);
      break;
    case EPI_UP_RELU:
      k_ffn_skinny<MT, 1, I8, EPI_UP_RELU, depth(MT, 1, I8), 4><<<grid, 256, 0, s>>>(a);
      break;
    case EPI_DOWN_ACC:
      k_ffn_skinny<MT, 1, I8, EPI_DOWN_ACC, depth(MT, 1, I8), 4><<<grid, 256, 0, s>>>(a);
      break;
    default:
      k_ffn_skinny<MT, 1, I8, EPI_DOWN_ROWS, depth(MT, 1, I8), 4><<<grid, 256, 0, s>>>(a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_skinny(const SkinnyArgs& a, int epi, bool i8, int mt, hipStream_t s) {
  if (i8) {
    if (mt <= 1) return launch_mt<1, true>(a, epi, s);
    if (mt == 2) return launch_mt<2, true>(a, epi, s);
    return launch_mt<4, true>(a, epi, s);
  }
  if (mt <= 1) return launch_mt<1, false>(a, epi, s);
  if (mt == 2) return launch_mt<2, false>(a, epi, s);
  return launch_mt<4, false>(a, epi, s);
}

}  // namespace moe
