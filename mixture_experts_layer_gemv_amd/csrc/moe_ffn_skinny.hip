// Expert FFN for decode-sized batches: a skinny grouped GEMM that streams each
// touched expert's weights from HBM once and multiplies them by that expert's
// few activation rows on the matrix cores.
//
// Design (prior art: the small-batch GEMM of the DeepSpeed-Inference summary,
// datalearner.com, section 3 "SBI-GeMM"):
//  - tiling along the output dimension: a workgroup owns CT 16-column tiles
//    of one expert (both SwiGLU streams of them), so the reduction stays
//    inside the workgroup (part 1 of that section).  When outputs are too few
//    to keep every CU streaming, the reduction dimension is also split over
//    workgroups (its two-kernel variant); the split partials meet in the fp32
//    atomic combine, so no second kernel is needed;
//  - SPLITK: the reduction is split over the workgroup's four waves and the
//    partial tiles meet in one LDS transpose, after which each thread reads
//    its outputs' partials contiguously (part 2, with wave64).  Otherwise each
//    wave owns CT neighbouring tiles over the whole reduction range and the
//    four waves load the same activation fragments at about the same time
//    (all but the first hit in L1), with no partial sums crossing waves.
//    Measured, the first is faster with one or two M tiles and the second
//    with four M tiles over packed activations;
//  - weights are re-laid out at initialisation so a wave's load is 1 KiB of
//    contiguous memory (part 3; see the packed layout in moe_kernels.hpp);
//  - small-batch work is bandwidth-bound, so the activations (a few rows per
//    expert) ride along in registers and the product runs on MFMA.
// Work items are (column tile, reduction slice, expert, row chunk) tuples
// generated on the device from the dispatch offsets: the host never reads the
// expert counts.  With `topk_idx` set, each workgroup derives the dispatch
// itself in its prologue (and logical workgroup 0 publishes it), so no
// separate dispatch launch is needed.
#include "moe_convert.hpp"
#include "moe_dispatch_block.hpp"
#include "moe_index.hpp"
#include "moe_lds.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// 16-byte load through a pointer the caller knows is in global memory.  The
// activation pointers pass through a per-tile array and a select, so the
// compiler cannot always infer their address space; a flat load then counts
// on both the vector-memory and the LDS counters and may complete out of
// order, which turns every wait on it into a full drain of the pipeline.
__device__ __forceinline__ u32x4_t load_global16(const uint16_t* p) {
  return *(const __attribute__((address_space(1))) u32x4_t*)p;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Waits until at most n units of STEP vector-memory operations each are
// outstanding; n is uniform, 0 <= n <= N.  (wait_units_nc: STEP = CG + nc for
// a uniform nc in [0, C].)
template <int STEP, int N>
__device__ __forceinline__ void wait_units(int n) {
  if constexpr (N <= 0) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  } else {
    if (n >= N)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(N * STEP));
    else
      wait_units<STEP, N - 1>(n);
  }
}
template <int CG, int C, int N>
__device__ __forceinline__ void wait_units_nc(int nc, int n) {
  if constexpr (C <= 0) {
    wait_units<CG, N>(n);
  } else {
    if (nc >= C)
      wait_units<CG + C, N>(n);
    else
      wait_units_nc<CG, C - 1, N>(nc, n);
  }
}

// Register plan of one variant: accumulators, registers per pipeline stage,
// and the deepest pipeline that fits 128 VGPRs (4 waves per SIMD) or else
// 256 VGPRs (2 waves per SIMD).
struct Plan {
  int acc, stage, wpe, depth;
};
constexpr Plan plan(int mt, int g, int ct, int qb, bool sa) {
  const int acc = ct * g * mt * 4;
  const int act = mt * q_ah(qb) * 4;  // one K unit of activations
  // with shared activations (sa) only the weights are in flight in
  // registers; the unit being consumed is read from LDS
  const int stage = ct * g * 4 + (qb == 5 ? ct * g : 0) + (sa ? 0 : act);
  // addresses, loop state, int8 conversion (and, shared, the unit read from LDS)
  // (int4 with per-wave activations: the converted weights of later units
  // are held too)
  const int fixed = (q_bits(qb) == 4 ? (sa ? 72 : 128) : (qb ? 64 : 40)) + (sa ? act + (qb ? 8 : 0) : 0);
  // shared activations: DA = depth + 1 units of the ring in at most 64 KiB,
  // so two workgroups fit a CU's LDS
  const int dmax0 = sa ? 64 / (mt * q_ah(qb)) - 1 : 6;
  const int dmax = dmax0 < 6 ? dmax0 : 6;
  const int d128 = (128 - fixed - acc) / stage;
  if (d128 >= 4) return Plan{acc, stage, 4, d128 < dmax ? d128 : dmax};
  const int d256 = (256 - fixed - acc) / stage;
  return Plan{acc, stage, 2, d256 < 2 ? 2 : (d256 < dmax ? d256 : dmax)};
}

typedef u32x4_t __attribute__((address_space(3))) lds_u32x4_t;

// Units of the shared-activation ring of one variant (16-byte lanes x 64).
constexpr int sa_ring_units(int mt, int g, int ct, int qb, bool sa) {
  return sa ? (plan(mt, g, ct, qb, sa).depth + 1) * mt * q_ah(qb) : 0;
}

// The dispatch offsets of a launch in LDS (offs_s[0..E]): read, or derived
// from topk_idx in every workgroup (DL then holds the histogram).
template <int NW>
__device__ __forceinline__ void skinny_offsets(const SkinnyArgs& A, DispatchLds<NW>& DL, int* offs_s) {
  const int tid = threadIdx.x;
  if (A.topk_idx) {
    block_histogram<NW>(A.topk_idx, A.T * A.topk, A.E, DL);
    if (tid <= A.E) offs_s[tid] = DL.offs[tid];
  } else {
    if (tid <= A.E) offs_s[tid] = A.offsets[tid];
  }
  __syncthreads();
}

// The (expert, chunk) pairs of R rows among the experts a launch admits, one
// lane per expert (E <= 64): its chunks, the pairs before it, and the total
// (skinny_pair's numbering, found without a serial walk over the experts).
struct PairScan {
  int nch, start, total;
};
__device__ __forceinline__ PairScan pair_scan(const SkinnyArgs& A, const int* offs_s, int R) {
  const int lane = threadIdx.x & 63;
  const int nch = lane < A.E ? pair_chunks(offs_s, lane, R, A.min_rows, A.max_rows) : 0;
  int incl = nch;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  return PairScan{nch, incl - nch, __builtin_amdgcn_readlane(incl, 63)};
}
// Expert and chunk of pair p (uniform); false if p is past the last pair.
__device__ __forceinline__ bool pair_find(const PairScan& ps, int p, int* e, int* chunk) {
  const unsigned long long m = __ballot(p >= ps.start && p < ps.start + ps.nch);
  if (m == 0) return false;
  const int l = __builtin_amdgcn_readfirstlane(__ffsll((long long)m) - 1);
  *e = l;
  *chunk = p - __builtin_amdgcn_readlane(ps.start, l);
  return true;
}

// Work items of one kind: column groups x reduction slices x pairs.
template <bool SPLITK, int CT>
__device__ __forceinline__ int skinny_items(const SkinnyArgs& A, const PairScan& ps) {
  const int NG = SPLITK ? A.N / 16 / CT : skinny_groups(A.N, CT);
  return NG * A.ksplit * ps.total;
}

// One workgroup's work: item wk (none unless `real`) over the pairs in ps.  offs_s: the offsets in LDS (skinny_offsets); publish: this
// workgroup writes the derived dispatch (with topk_idx).  sa_ring: the
// workgroup's shared-activation ring, at least sa_ring_units() KiB (unused
// otherwise).
template <int MT, int G, int CT, int QB, int EPI, int NW, bool SPLITK, bool SA>
__device__ __forceinline__ void skinny_body(const SkinnyArgs& A, const SkinnyWork& wk, bool real, const PairScan& ps,
                                            bool publish, const int* offs_s, DispatchLds<NW>& DL,
                                            lds_u32x4_t* sa_ring) {
  static_assert(!(SA && SPLITK), "shared activations need every wave on the same K range");
  constexpr int D = plan(MT, G, CT, QB, SA).depth;
  constexpr int R = 16 * MT;        // rows per work item
  constexpr int AH = q_ah(QB);  // activation loads per K unit
  constexpr int UK = 32 * AH;   // k per unit
  // Shared activations: the NAF activation fragments of a K unit are copied
  // once per workgroup into an LDS ring of DA units (wave w copies fragments
  // w, w + NW, ...: NC of them, at most CPW; waves past NAF copy none) and
  // every wave reads them there.  Only the fragments holding real rows are
  // copied; the slots of the others keep stale data, which feeds only
  // accumulator rows that are never stored.
  constexpr int NAF = MT * AH;
  constexpr int CPW = (NAF + NW - 1) / NW;  // most copies per wave per unit
  constexpr int DA = D + 1;
  constexpr int CG = CT * G;  // weight loads per unit and wave
  static_assert(!SA || (D - 1) * (CG + CPW) <= 63, "vmcnt holds at most 63");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  __shared__ int rows_s[R];

  const int NB = A.N / 16;  // a multiple of 4 (N is a multiple of 64)
  const int S = A.ksplit;
  // first of this wave's CT column tiles (the workgroup's, with SPLITK)
  const int ntile = SPLITK ? wk.ngroup * CT : (wk.ngroup * NW + wave) * CT;
  const int ks = wk.ks;
  const int n_assign = A.T * A.topk;

  // (expert, chunk) of this work item
  int e = 0, chunk = 0;
  const bool has_pair = real && pair_find(ps, wk.pair, &e, &chunk);
  const bool valid = wk.ngroup * (SPLITK ? 1 : NW) * CT < NB && has_pair;
  const int row0 = valid ? offs_s[e] + chunk * R : 0;
  const int nrows = valid ? min(R, offs_s[e + 1] - row0) : 0;

  if (A.topk_idx) {
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
  // (NB is a multiple of 4, so a wave's tiles are all in or all out.)  With
  // shared activations a wave past the last tile stays for the copies and
  // barriers, streaming the group's first tiles, and stores nothing.
  const bool live = ntile < NB;
  if (!SA && !live) return;
  const int ltile = live ? ntile : wk.ngroup * NW * CT;

  // Activation pointers of this lane, one per M tile, and the element strides
  // of a K unit (su) and of its second 32-k half for int8 (sh).
  //  - packed rows (moe_index.hpp layout): the chunk's M tile mt is the 1 KiB
  //    fragment row (prow0/16 + mt), one contiguous load per K unit; tiles
  //    past the chunk's last real row re-read its last fragment;
  //  - row-major rows: lane l reads 16 bytes of row (l mod 16) of the tile,
  //    gathered through the dispatch for the up projection; lanes past the
  //    chunk's last row read the chunk's first row.
  // Either way every load is unconditional and the extra rows are never
  // stored.
  const int prow0 = A.packed || A.h_packed ? padded_offset(offs_s, e) + chunk * R : 0;
  const uint16_t* arow[MT];
  int su, sh;
  if (A.packed) {
    const int nfrag = (nrows + 15) >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      arow[mt] = A.act + ((size_t)(prow0 >> 4) + min(mt, nfrag - 1)) * (A.K / 32) * 512 + 8 * lane;
    su = AH * 512;
    sh = 512;
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = mt * 16 + (lane & 15);
      const int rr = r < nrows ? r : 0;
      const int src = A.gather ? rows_s[rr] / A.topk : row0 + rr;
      arow[mt] = A.act + (size_t)src * A.K + 8 * (lane >> 4);
    }
    su = UK;
    sh = 32;
  }

  const int U = A.K / UK;
  int u0, u1;
  if constexpr (SPLITK)
    unit_range(ks * NW + wave, S * NW, U, &u0, &u1);
  else
    unit_range(ks, S, U, &u0, &u1);
  // the CT column tiles of this group are consecutive streams of U*G units
  const u32x4_t* wp = static_cast<const u32x4_t*>(A.w) + (size_t)(e * NB + ltile) * U * G * 64 + lane;
  const size_t tile_stride = (size_t)U * G * 64;

  floatx4_t acc[CT][G][MT];
  floatx4_t acc_x[QB == 4 ? MT : 1];  // int4: sum of the activations over the K range, per row
#pragma unroll
  for (int mt = 0; mt < (QB == 4 ? MT : 1); ++mt) acc_x[mt] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[c][g][mt] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4_t wb[D][CT][G];
  uint32_t sbw[QB == 5 ? D : 1][CT][G];  // MXFP4: the lane's column's block scales of a unit (byte h: step h)
  const uint32_t* const mxp = QB == 5 ? A.mx + (size_t)(e * NB + ltile) * U * G * 16 + (lane & 15) : nullptr;
  const size_t mx_tile_stride = (size_t)U * G * 16;
  u32x4_t ab[SA ? 1 : D][MT][AH];

  // Shared activations: this wave's copies (fragment, uniform source of
  // unit 0) and the ring.  Packed rows only: tiles past the chunk's last
  // real row re-read its last fragment, as the per-wave loads do.
  const char* sa_src[CPW];
  int sa_frag[CPW];
  const uint32_t sa_lds = (uint32_t)(uintptr_t)sa_ring;
  int NC = 0;  // this wave's copies per unit (uniform)
  if constexpr (SA) {
    const int rb = __builtin_amdgcn_readfirstlane(prow0 >> 4);
    const int nfrag = __builtin_amdgcn_readfirstlane((nrows + 15) >> 4);
    const int naf = min(NAF, nfrag * AH);  // fragments holding real rows
    NC = wave < naf ? (naf - 1 - wave) / NW + 1 : 0;
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int f = min(wave + NW * j, NAF - 1);  // (used only for j < NC)
      const int mt = f / AH, h = f % AH;
      sa_frag[j] = f;
      sa_src[j] = reinterpret_cast<const char*>(A.act + ((size_t)(rb + min(mt, nfrag - 1)) * (A.K / 32) + h) * 512);
    }
  }

#define MOE_ISSUE(slot, u)                                                                             \
  do {                                                                                                 \
    _Pragma("unroll") for (int c = 0; c < CT; ++c) _Pragma("unroll") for (int g = 0; g < G; ++g)      \
        wb[slot][c][g] = __builtin_nontemporal_load(wp + c * tile_stride + ((size_t)(u) * G + g) * 64); \
    if constexpr (QB == 5) {                                                                           \
      _Pragma("unroll") for (int c = 0; c < CT; ++c) _Pragma("unroll") for (int g = 0; g < G; ++g)    \
          sbw[slot % (QB == 5 ? D : 1)][c][g] =                                                       \
              __builtin_nontemporal_load(mxp + c * mx_tile_stride + ((size_t)(u) * G + g) * 16);      \
    }                                                                                                  \
    if constexpr (SA) {                                                                                \
      _Pragma("unroll") for (int j = 0; j < CPW; ++j) if (j < NC)                                      \
          copy_frag(sa_src[j] + (size_t)(u) * (AH * 1024), 16u * lane,                                 \
                    sa_lds + (uint32_t)((((u) % DA) * NAF + sa_frag[j]) * 1024));                      \
    } else {                                                                                           \
      _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) _Pragma("unroll") for (int h = 0; h < AH; ++h) \
          ab[slot][mt][h] = load_global16(arow[mt] + (size_t)(u) * su + sh * h);                       \
    }                                                                                                  \
  } while (0)

  // Activations of the unit being consumed.  Shared: wait until at most
  // `after` later units of this wave's operations are outstanding (its
  // copies of this unit have landed), pass the barrier (so have every
  // wave's), then read the unit's fragments from the ring.
#define MOE_ACT_FETCH(slot, u, after)                                                                  \
  u32x4_t av[SA ? MT : 1][AH];                                                                         \
  if constexpr (SA) {                                                                                  \
    wait_units_nc<CG, CPW, D - 1>(NC, after);                                                          \
    ring_barrier();                                                                                    \
    const lds_u32x4_t* st_ = sa_ring + ((u) % DA) * NAF * 64 + lane;                                   \
    _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) _Pragma("unroll") for (int h = 0; h < AH; ++h)   \
        av[mt][h] = st_[(mt * AH + h) * 64];                                                           \
  }
#define MOE_ACT(slot, mt, h) (SA ? av[(mt) % (SA ? MT : 1)][h] : ab[(slot) % (SA ? 1 : D)][mt][h])

#define MOE_CONSUME(slot, u, after)                                                                    \
  do {                                                                                                 \
    MOE_ACT_FETCH(slot, u, after)                                                                      \
    _Pragma("unroll") for (int c = 0; c < CT; ++c) {                                                   \
      if constexpr (QB == 8 || QB == 9) {                                                              \
        _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                                \
          _Pragma("unroll") for (int g = 0; g < G; ++g) {                                              \
            const u32x4_t q = wb[slot][c][g];                                                          \
            const bf16x8_t bw = QB == 9 ? (h == 0 ? fp8x8_to_bf16(q[0], q[1]) : fp8x8_to_bf16(q[2], q[3])) \
                                        : (h == 0 ? i8x8_to_bf16(q[0], q[1]) : i8x8_to_bf16(q[2], q[3])); \
            _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) acc[c][g][mt] =                          \
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(MOE_ACT(slot, mt, h)), bw, acc[c][g][mt], 0, 0, 0); \
          }                                                                                            \
        }                                                                                              \
      } else if constexpr (QB == 5) {                                                                  \
        _Pragma("unroll") for (int h = 0; h < 4; ++h) {                                                \
          _Pragma("unroll") for (int g = 0; g < G; ++g) {                                              \
            const bf16x8_t bw = fp4x8_to_bf16(wb[slot][c][g][h], e8m0_at(sbw[slot % (QB == 5 ? D : 1)][c][g], h)); \
            _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) acc[c][g][mt] =                          \
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(MOE_ACT(slot, mt, h)), bw, acc[c][g][mt], 0, 0, 0); \
          }                                                                                            \
        }                                                                                              \
      } else if constexpr (QB == 4) {                                                                  \
        _Pragma("unroll") for (int h = 0; h < 4; ++h) {                                                \
          if (c == 0) {                                                                                \
            const bf16x8_t ones = as_bf16x8(u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}); \
            _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) acc_x[mt] =                              \
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(MOE_ACT(slot, mt, h)), ones, acc_x[mt], 0, 0, 0); \
          }                                                                                            \
          _Pragma("unroll") for (int g = 0; g < G; ++g) {                                              \
            const bf16x8_t bw = u4x8_to_bf16_biased(wb[slot][c][g][h]);                                \
            _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) acc[c][g][mt] =                          \
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(MOE_ACT(slot, mt, h)), bw, acc[c][g][mt], 0, 0, 0); \
          }                                                                                            \
        }                                                                                              \
      } else {                                                                                         \
        _Pragma("unroll") for (int g = 0; g < G; ++g) {                                                \
          const bf16x8_t bw = as_bf16x8(wb[slot][c][g]);                                               \
          _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) acc[c][g][mt] =                            \
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(MOE_ACT(slot, mt, 0)), bw, acc[c][g][mt], 0, 0, 0); \
        }                                                                                              \
      }                                                                                                \
    }                                                                                                  \
  } while (0)

  // Software pipeline, D units in flight.  When the wave has at least 2D
  // units: an unguarded prologue and steady state (straight-line code, so the
  // compiler waits only for the unit being consumed), then a guarded tail of
  // fewer than 2D units.  Short reductions take a plain loop.  The third
  // argument of MOE_CONSUME is the number of later units already issued
  // (the shared-activation wait depends on it).
  if (u1 - u0 >= 2 * D) {
#pragma unroll
    for (int d = 0; d < D; ++d) MOE_ISSUE(d, u0 + d);
    int u = u0;
    for (; u + 2 * D <= u1; u += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        MOE_CONSUME(d, u + d, D - 1);
        MOE_ISSUE(d, u + d + D);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (u + d < u1) {
        MOE_CONSUME(d, u + d, min(D - 1, u1 - 1 - (u + d)));
        if (u + d + D < u1) MOE_ISSUE(d, u + d + D);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (u + D + d < u1) MOE_CONSUME(d, u + D + d, u1 - 1 - (u + D + d));
  } else {
    for (int u = u0; u < u1; ++u) {
      MOE_ISSUE(0, u);
      MOE_CONSUME(0, u, 0);
    }
  }
#undef MOE_CONSUME
#undef MOE_ACT
#undef MOE_ACT_FETCH
#undef MOE_ISSUE
  if constexpr (QB == 4) {  // remove the weights' bias: acc holds sum x (q + 136)
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[c][g][mt][i] = fmaf(-kI4Bias, acc_x[mt][i], acc[c][g][mt][i]);
  }
  if (!live) return;  // (shared activations only: other waves past NB returned above)

  // Stores one output element (row of the chunk, column) from its G sums.
  auto store = [&](int row, int col, const float* v) {
    const int r = row0 + row;
    if constexpr (EPI == EPI_UP_SWIGLU) {
      float gv = v[0], uv = v[G - 1];
      if constexpr (q_chan_scale(QB)) {
        gv *= A.scale0[(size_t)e * A.N + col];
        uv *= A.scale1[(size_t)e * A.N + col];
      }
      A.h_out[A.h_packed ? packed_index(prow0 + row, col, A.N) : (size_t)r * A.N + col] =
          f32_to_bf16(silu(gv) * uv);
    } else if constexpr (EPI == EPI_UP_RELU) {
      float gv = v[0];
      if constexpr (q_chan_scale(QB)) gv *= A.scale0[(size_t)e * A.N + col];
      A.h_out[A.h_packed ? packed_index(prow0 + row, col, A.N) : (size_t)r * A.N + col] =
          f32_to_bf16(gv > 0.0f ? gv : 0.0f);
    } else {
      float o2 = v[0];
      if constexpr (q_chan_scale(QB)) o2 *= A.scale0[(size_t)e * A.N + col];
      if constexpr (EPI == EPI_DOWN_ACC) {
        const int a = A.perm[r];
        unsafeAtomicAdd(A.f_out + (size_t)(a / A.topk) * A.N + col, A.topk_w[a] * o2);
      } else {  // unweighted row, this reduction slice's partial sum
        A.f_out[(size_t)ks * A.slice_stride + (size_t)r * A.N + col] = o2;
      }
    }
  };

  // Lane l of tile (c, g, mt) holds rows mt*16 + 4*(l>>4) + i, i = 0..3, of
  // column (ntile + c)*16 + (l & 15).
  if constexpr (SPLITK) {
    // Cross-wave reduction through one LDS transpose: wave w writes its
    // partial tiles; each output's NW partials are then read by one thread.
    __shared__ float red[NW * CT * G * MT * 256];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            red[(((wave * CT + c) * G + g) * MT + mt) * 256 + i * 64 + lane] = acc[c][g][mt][i];
    __syncthreads();
    for (int o = tid; o < CT * MT * 256; o += NW * 64) {
      const int c = o / (MT * 256), mt = (o >> 8) % MT, i = (o >> 6) & 3, ln = o & 63;
      const int row = mt * 16 + 4 * (ln >> 4) + i;
      if (row >= nrows) continue;
      float v[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += red[(((w * CT + c) * G + g) * MT + mt) * 256 + i * 64 + ln];
        v[g] = sum;
      }
      store(row, (ntile + c) * 16 + (ln & 15), v);
    }
  } else {
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mt * 16 + 4 * (lane >> 4) + i;
          if (row >= nrows) continue;
          float v[G];
#pragma unroll
          for (int g = 0; g < G; ++g) v[g] = acc[c][g][mt][i];
          store(row, (ntile + c) * 16 + (lane & 15), v);
        }
  }
}

// Block b takes logical item xcd_logical(b) of the upper-bound grid (the
// padding pairs past the last real one interleaved, so none of them is left
// for the end of a many-round launch); block 0 publishes the derived
// dispatch.
template <int MT, int G, int CT, int QB, int EPI, int NW, bool SPLITK, bool SA>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(plan(MT, G, CT, QB, SA).wpe))) void
k_ffn_skinny(const SkinnyArgs A) {
  constexpr int units = sa_ring_units(MT, G, CT, QB, SA);
  __shared__ __attribute__((aligned(16))) u32x4_t ring[units > 0 ? units * 64 : 1];
  __shared__ DispatchLds<NW> DL;
  __shared__ int offs_s[kMaxExperts + 1];
  skinny_offsets<NW>(A, DL, offs_s);
  const PairScan ps = pair_scan(A, offs_s, 16 * MT);
  skinny_body<MT, G, CT, QB, EPI, NW, SPLITK, SA>(A, skinny_work(xcd_logical(blockIdx.x, gridDim.x), A.W, A.ksplit),
                                                  true, ps, blockIdx.x == 0, offs_s, DL, (lds_u32x4_t*)ring);
}

// A projection split by expert size in one launch: the twelve-tile items of
// the experts above one four-tile chunk and the four-tile items of the
// others.  Every XCD starts its share of the twelve-tile items first (the
// longest), then its four-tile items, then the grid's padding (xcd_item): a
// launch of about one round, whose placement a padding block taking a slot
// early would unbalance (measured: 33 CUs with one workgroup and 33 with
// three on the skewed layer's down projection, -8 us with this order).  Both kinds
// stream 2 KiB of weights per wave and K unit (one column tile of gate and
// up, or two of ReLU), so the blocks are of one size and the launch's last
// round stays short.  Both kinds share one ring allocation; the launch runs
// at two waves per SIMD (the twelve-tile variant's budget).
constexpr int split_ct(int g) { return g == 2 ? 1 : 2; }

template <int G, int EPI, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_ffn_skinny_split(
    const SkinnyArgs AN, const SkinnyArgs AW) {
  constexpr int CT = split_ct(G);
  constexpr int uw = sa_ring_units(12, G, CT, 0, true), un = sa_ring_units(4, G, CT, 0, true);
  __shared__ __attribute__((aligned(16))) u32x4_t ring[(uw > un ? uw : un) * 64];
  __shared__ DispatchLds<NW> DL;
  __shared__ int offs_s[kMaxExperts + 1];
  skinny_offsets<NW>(AN, DL, offs_s);  // (packed rows: read, never derived)
  const PairScan pw = pair_scan(AW, offs_s, 16 * 12), pn = pair_scan(AN, offs_s, 16 * 4);
  const int nw = skinny_items<false, CT>(AW, pw), nn = skinny_items<false, CT>(AN, pn);
  const int item = xcd_item(blockIdx.x, nw, nn);
  if (item >= 0 && item < nw)
    skinny_body<12, G, CT, 0, EPI, NW, false, true>(AW, skinny_work(item, max(pw.total, 1), 1), true, pw, false, offs_s,
                                                        DL, (lds_u32x4_t*)ring);
  else
    skinny_body<4, G, CT, 0, EPI, NW, false, true>(AN, skinny_work(item < 0 ? 0 : item - nw, max(pn.total, 1), 1),
                                                       item >= 0, pn, false, offs_s, DL, (lds_u32x4_t*)ring);
}

// One variant; variants whose accumulators exceed the register budget are
// never built (the host does not ask for them).
template <int MT, int G, int CT, int QB, int EPI, bool SPLITK, bool SA>
hipError_t launch_one(const SkinnyArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (CT * G * MT * 4 > 96) {
    return hipErrorInvalidValue;
  } else {
    k_ffn_skinny<MT, G, CT, QB, EPI, 4, SPLITK, SA><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
  }
}

template <int MT, int CT, int QB, bool SPLITK, bool SA>
hipError_t launch_ct(const SkinnyArgs& a, int epi, hipStream_t s) {
  const int NG = SPLITK ? a.N / 16 / CT : skinny_groups(a.N, CT);
  const long long work = (long long)NG * a.W * a.ksplit;
  const long long nblk = (work + 7) / 8 * 8;
  const dim3 grid((unsigned)nblk);
  switch (epi) {
    case EPI_UP_SWIGLU:
      if constexpr (q_bits(QB) == 4 && MT == 2 && CT == 4 && !SA) {  // (would spill: two tiles instead)
        return launch_ct<MT, 2, QB, SPLITK, SA>(a, epi, s);
      } else {
        return launch_one<MT, 2, CT, QB, EPI_UP_SWIGLU, SPLITK, SA>(a, grid, s);
      }
    case EPI_UP_RELU: return launch_one<MT, 1, CT, QB, EPI_UP_RELU, SPLITK, SA>(a, grid, s);
    case EPI_DOWN_ACC: return launch_one<MT, 1, CT, QB, EPI_DOWN_ACC, SPLITK, SA>(a, grid, s);
    default: return launch_one<MT, 1, CT, QB, EPI_DOWN_ROWS, SPLITK, SA>(a, grid, s);
  }
}

// Shared activations only where the waves of a workgroup share a K range
// (columns split over the waves) and the rows are packed; twelve M tiles
// exist only in that form.
template <int MT, int CT, int QB, bool SPLITK>
hipError_t launch_sa(const SkinnyArgs& a, int epi, hipStream_t s) {
  if constexpr (!SPLITK) {
    if (a.shared_act) return launch_ct<MT, CT, QB, SPLITK, true>(a, epi, s);
  }
  if constexpr (MT > 4) {
    return hipErrorInvalidValue;
  } else {
    return launch_ct<MT, CT, QB, SPLITK, false>(a, epi, s);
  }
}

template <int MT, int QB, bool SPLITK>
hipError_t launch_mt(const SkinnyArgs& a, int epi, int ct, hipStream_t s) {
  if constexpr (MT < 4) {
    if (ct >= 4) return launch_sa<MT, 4, QB, SPLITK>(a, epi, s);
  }
  if (ct >= 2) return launch_sa<MT, 2, QB, SPLITK>(a, epi, s);
  return launch_sa<MT, 1, QB, SPLITK>(a, epi, s);
}

template <bool SPLITK>
hipError_t launch_split(const SkinnyArgs& a, int epi, int qb, int mt, int ct, hipStream_t s) {
  if (qb == 8) {  // int8 stops at two M tiles: four spill registers
    if (mt <= 1) return launch_mt<1, 8, SPLITK>(a, epi, ct, s);
    return launch_mt<2, 8, SPLITK>(a, epi, ct, s);
  }
  if (qb == 9) {  // fp8: as int8
    if (mt <= 1) return launch_mt<1, 9, SPLITK>(a, epi, ct, s);
    return launch_mt<2, 9, SPLITK>(a, epi, ct, s);
  }
  if (qb == 4) {  // int4: as int8
    if (mt <= 1) return launch_mt<1, 4, SPLITK>(a, epi, ct, s);
    return launch_mt<2, 4, SPLITK>(a, epi, ct, s);
  }
  if (qb == 5) {  // MXFP4: as int4
    if (mt <= 1) return launch_mt<1, 5, SPLITK>(a, epi, ct, s);
    return launch_mt<2, 5, SPLITK>(a, epi, ct, s);
  }
  if (mt <= 1) return launch_mt<1, 0, SPLITK>(a, epi, ct, s);
  if (mt == 2) return launch_mt<2, 0, SPLITK>(a, epi, ct, s);
  if (mt <= 4) return launch_mt<4, 0, SPLITK>(a, epi, ct, s);
  if constexpr (SPLITK) {
    return hipErrorInvalidValue;
  } else {
    return launch_mt<12, 0, SPLITK>(a, epi, ct, s);
  }
}

}  // namespace

hipError_t launch_ffn_skinny_split(const SkinnyArgs& narrow, const SkinnyArgs& wide, int epi, hipStream_t s) {
  if (!narrow.shared_act || !wide.shared_act || !narrow.packed || !wide.packed) return hipErrorInvalidValue;
  if (narrow.ksplit != 1 || wide.ksplit != 1) return hipErrorInvalidValue;
  const int G = epi == EPI_UP_SWIGLU ? 2 : 1;
  constexpr int NW = 4;  // (8 waves sharing one ring measured slower on the skewed layer)
  // each kind's upper bound on items, rounded up per XCD (xcd_item)
  auto blocks = [&](const SkinnyArgs& x, int ct) {
    const int tiles = NW * ct;
    const long long work = (long long)((x.N / 16 + tiles - 1) / tiles) * x.W;
    return (work + 7) / 8 * 8;
  };
  const long long nw = blocks(wide, split_ct(G)), nn = blocks(narrow, split_ct(G));
  if (nw + nn > 0x7FFFFFF0LL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(nw + nn));
  switch (epi) {
    case EPI_UP_SWIGLU: k_ffn_skinny_split<2, EPI_UP_SWIGLU, NW><<<grid, NW * 64, 0, s>>>(narrow, wide); break;
    case EPI_UP_RELU: k_ffn_skinny_split<1, EPI_UP_RELU, NW><<<grid, NW * 64, 0, s>>>(narrow, wide); break;
    case EPI_DOWN_ACC: k_ffn_skinny_split<1, EPI_DOWN_ACC, NW><<<grid, NW * 64, 0, s>>>(narrow, wide); break;
    default: k_ffn_skinny_split<1, EPI_DOWN_ROWS, NW><<<grid, NW * 64, 0, s>>>(narrow, wide); break;
  }
  return hipGetLastError();
}

hipError_t launch_ffn_skinny(const SkinnyArgs& a, int epi, int qb, int mt, int ct, bool splitk, hipStream_t s) {
  if (qb != 0 && qb != 8 && qb != 9 && qb != 4 && qb != 5) return hipErrorInvalidValue;
  if (qb == 5 && !a.mx) return hipErrorInvalidValue;
  if (a.shared_act && (splitk || !a.packed)) return hipErrorInvalidValue;
  if (mt > 4 && (mt != 12 || qb || splitk || !a.shared_act)) return hipErrorInvalidValue;
  return splitk ? launch_split<true>(a, epi, qb, mt, ct, s) : launch_split<false>(a, epi, qb, mt, ct, s);
}

}  // namespace moe
