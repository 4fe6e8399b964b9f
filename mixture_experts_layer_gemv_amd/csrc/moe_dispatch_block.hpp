// Block-level expert dispatch shared by the dispatch kernel and the decode
// FFN prologue: histogram of expert ids in LDS, exclusive prefix sum, and the
// stable position of every assignment (expert-major, increasing assignment id
// inside an expert).  Within a wave, lanes holding the same expert find each
// other with six ballots (one per bit of the id, E <= 64) and rank by lane
// order; across waves a per-expert running cursor orders the waves.
#pragma once

#include "moe_kernels.hpp"

namespace moe {

template <int NW>
struct DispatchLds {
  int cnt[64];
  int offs[65];
  int cursor[64];
  int wbase[NW][64];
};

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// counts -> L.cnt, exclusive offsets -> L.offs (offs[E] = n).  All threads call.
template <int NW>
__device__ void block_histogram(const int32_t* __restrict__ idx, int n, int E, DispatchLds<NW>& L) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    L.cnt[tid] = 0;
    L.cursor[tid] = 0;
  }
  __syncthreads();
  for (int a = tid; a < n; a += NW * 64) atomicAdd(&L.cnt[clamp_expert(idx[a], E)], 1);
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
}

// Calls fn(a, e, pos) for every assignment a in [lo, hi) with its stable
// position pos.  Needs L.offs (the experts' first positions) and L.cursor (per
// expert, the assignments before lo that it holds); advances L.cursor past
// hi.  All threads call.
template <int NW, class F>
__device__ void block_stable_positions_range(const int32_t* __restrict__ idx, int lo, int hi, int E,
                                             DispatchLds<NW>& L, F&& fn) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (long long base = lo; base < hi; base += NW * 64) {  // 64-bit: hi may be near 2^31
    const bool valid = base + tid < hi;
    const int a = valid ? (int)(base + tid) : 0;
    const int e = valid ? clamp_expert(idx[a], E) : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 6; ++b) {
      const uint64_t mb = __ballot((e >> b) & 1);
      peers &= ((e >> b) & 1) ? mb : ~mb;
    }
    const int rank = __popcll(peers & lt);
    L.wbase[wave][lane] = 0;
    __syncthreads();
    if (valid && rank == 0) L.wbase[wave][e] = __popcll(peers);
    __syncthreads();
    if (tid < E) {
      int run = L.cursor[tid];
      for (int w = 0; w < NW; ++w) {
        const int c = L.wbase[w][tid];
        L.wbase[w][tid] = run;
        run += c;
      }
      L.cursor[tid] = run;
    }
    __syncthreads();
    if (valid) fn(a, e, L.offs[e] + L.wbase[wave][e] + rank);
    __syncthreads();
  }
}

// Calls fn(a, e, pos) for every assignment a with its stable position pos.
// Needs block_histogram first; leaves L.cursor at the counts.  All threads call.
template <int NW, class F>
__device__ void block_stable_positions(const int32_t* __restrict__ idx, int n, int E, DispatchLds<NW>& L, F&& fn) {
  block_stable_positions_range<NW>(idx, 0, n, E, L, static_cast<F&&>(fn));
}

}  // namespace moe
