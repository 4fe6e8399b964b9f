// Index arithmetic of the decode FFN launch, shared by the kernel and a host
// test that checks it exhaustively.  No HIP dependency, so a plain C++
// compiler can build it.
#pragma once

#if defined(__HIPCC__) || defined(__HIP__)
#define MOE_HD __host__ __device__
#else
#define MOE_HD
#endif

namespace moe {

// Workgroups are dealt to the 8 XCDs round-robin (b -> XCD b % 8).  This
// renumbering gives each XCD a contiguous range of logical indices, so work
// items with neighbouring logical indices share that XCD's L2.
// nblk must be a multiple of 8.
MOE_HD inline int xcd_logical(int b, int nblk) { return (b & 7) * (nblk >> 3) + (b >> 3); }

// Logical index -> (column-tile group, reduction slice, (expert, chunk) pair),
// pair fastest, for W pairs and S slices per group.
struct SkinnyWork {
  int ngroup, ks, pair;
};

MOE_HD inline SkinnyWork skinny_work(int L, int W, int S) {
  SkinnyWork w;
  w.ngroup = L / (W * S);
  const int rem = L - w.ngroup * (W * S);
  w.ks = rem / W;
  w.pair = rem - w.ks * W;
  return w;
}

// The pair-th (expert, row chunk) in expert order, chunks of R rows, given
// dispatch offsets[0..E].  Returns false when pair is past the last chunk.
// npairs receives the total number of chunks.
MOE_HD inline bool skinny_pair(const int* offsets, int E, int R, int pair, int* e, int* chunk, int* npairs) {
  int n = 0;
  *e = -1;
  *chunk = 0;
  for (int i = 0; i < E; ++i) {
    const int nch = (offsets[i + 1] - offsets[i] + R - 1) / R;
    if (*e < 0 && pair >= n && pair < n + nch) {
      *e = i;
      *chunk = pair - n;
    }
    n += nch;
  }
  *npairs = n;
  return *e >= 0;
}

// Reduction units [u0, u1) of slice `part` out of `parts` for U units.
MOE_HD inline void unit_range(int part, int parts, int U, int* u0, int* u1) {
  *u0 = (int)(((long long)part * U) / parts);
  *u1 = (int)(((long long)(part + 1) * U) / parts);
}

}  // namespace moe
