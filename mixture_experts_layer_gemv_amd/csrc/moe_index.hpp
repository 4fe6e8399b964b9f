// Index arithmetic of the FFN launches, shared by the kernels and a host test
// that checks it exhaustively.  No HIP dependency, so a plain C++
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

// Grouped GEMM.  Logical workgroup -> (column block, (expert, row block)
// pair), pair fastest, for W pairs.
struct GemmWork {
  int nblock, mpair;
};

MOE_HD inline GemmWork gemm_work(int L, int W) {
  GemmWork w;
  w.nblock = L / W;
  w.mpair = L - w.nblock * W;
  return w;
}

// Byte offset of the 16 bytes lane `lane` copies for B fragment `bi` of a
// workgroup's stage, at reduction unit 0 (unit u adds u * G * 1 KiB).  The
// workgroup's fragments are ordered wave column major, nf per wave column,
// G fragments (gate, up) per 16-column tile; tiles past NB-1 re-read tile
// NB-1 so a partial column block never leaves the projection.
MOE_HD inline unsigned long long gemm_b_offset(int e, int NB, int U, int G, int tile_base, int nf, int bi,
                                               int lane) {
  const int f = bi % nf;
  int nb = tile_base + (bi / nf) * (nf / G) + f / G;
  nb = nb < NB ? nb : NB - 1;
  return ((unsigned long long)(e * NB + nb) * U * G + f % G) * 1024ull + 16ull * lane;
}

// Byte offset of lane `lane`'s 16 bytes of an A fragment whose rows start at
// activation row `row` (bf16, K per row), at reduction unit 0 (unit u adds
// 64 bytes).
MOE_HD inline unsigned long long gemm_a_offset(int row, int K, int lane) {
  return (unsigned long long)row * K * 2ull + 16ull * (lane >> 4);
}

}  // namespace moe
