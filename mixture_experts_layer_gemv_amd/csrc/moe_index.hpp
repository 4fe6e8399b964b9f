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

// Workgroups are dealt to the 8 XCDs round-robin (blocks b with one value of
// b % 8 run on one XCD).  This renumbering gives each XCD a contiguous range
// of logical indices, so work items with neighbouring logical indices share
// that XCD's L2.  nblk must be a multiple of 8.
MOE_HD inline int xcd_logical(int b, int nblk) { return (b & 7) * (nblk >> 3) + (b >> 3); }

// The same for launches whose grid is an upper bound on the work: n0 items of
// kind 0 and n1 of kind 1 (known only on the device), each kind's range cut
// into 8 contiguous parts, one per XCD.  The XCD's j-th block (b = 8 j + x)
// takes its part of kind 0, then its part of kind 1, then is padding (-1):
// in dispatch order every XCD starts all its real items before any padding
// block, so padding never holds a slot that a real item is waiting for.
// Items n0.. are kind 1.  Over all blocks of a grid with at least
// ceil(n0 / 8) + ceil(n1 / 8) blocks per XCD every item comes out exactly
// once.
MOE_HD inline int xcd_item(int b, int n0, int n1) {
  const int x = b & 7;
  const unsigned j = (unsigned)b >> 3;
  const int a0 = (int)((long long)x * n0 / 8), b0 = (int)((long long)(x + 1) * n0 / 8);
  const int a1 = (int)((long long)x * n1 / 8), b1 = (int)((long long)(x + 1) * n1 / 8);
  if (j < (unsigned)(b0 - a0)) return a0 + (int)j;
  if (j < (unsigned)(b0 - a0 + b1 - a1)) return n0 + a1 + (int)(j - (unsigned)(b0 - a0));
  return -1;
}

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

// Column groups of the decode FFN launch: each workgroup's 4 waves own CT
// consecutive 16-column tiles each.  Wave w of group g owns tiles
// (4 g + w) CT .. +CT-1; with N a multiple of 64 and CT in {1, 2, 4} a wave's
// tiles are either all below N/16 or all past it.
MOE_HD inline int skinny_groups(int N, int CT) { return (N / 16 + 4 * CT - 1) / (4 * CT); }

// Row chunks of expert e admitted by the window (min_rows, max_rows] (a bound
// <= 0 is absent): the pairs skinny_pair counts for e.  The kernels give each
// expert a lane and take a prefix sum of these across the wave.
MOE_HD inline int pair_chunks(const int* offsets, int e, int R, int min_rows = 0, int max_rows = 0) {
  const int cnt = offsets[e + 1] - offsets[e];
  const bool in = (min_rows <= 0 || cnt > min_rows) && (max_rows <= 0 || cnt <= max_rows);
  return in ? (cnt + R - 1) / R : 0;
}

// The pair-th (expert, row chunk) in expert order, chunks of R rows, given
// dispatch offsets[0..E], counting only experts whose row count lies in
// (min_rows, max_rows] (a bound <= 0 is absent).  Returns false when pair is
// past the last chunk.  npairs receives the total number of chunks.
MOE_HD inline bool skinny_pair(const int* offsets, int E, int R, int pair, int* e, int* chunk, int* npairs,
                               int min_rows = 0, int max_rows = 0) {
  int n = 0;
  *e = -1;
  *chunk = 0;
  for (int i = 0; i < E; ++i) {
    const int nch = pair_chunks(offsets, i, R, min_rows, max_rows);
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

// Grouped GEMM work order.  Logical workgroup L -> (expert e, row block mb,
// column block nblock): experts in turn; within an expert, groups of CG
// column blocks; within a group, each row block across the group's column
// blocks.  Consecutive logical indices run together on one XCD, so the
// workgroups resident at once share both their activation rows and their
// weight panels in that XCD's L2.  BM rows per row block, NBL column blocks;
// experts with fewer than min_rows rows get no work (another kernel serves
// them).  Returns false for logical indices past the last item (grid
// padding).
// The number of (expert, row block, column block) items of that work order.
MOE_HD inline int gemm_items(const int* offsets, int E, int BM, int NBL) {
  int w = 0;
  for (int i = 0; i < E; ++i) w += (offsets[i + 1] - offsets[i] + BM - 1) / BM * NBL;
  return w;
}

MOE_HD inline bool gemm_item(const int* offsets, int E, int BM, int NBL, int CG, int L, int* e, int* mb,
                             int* nblock, int min_rows = 1) {
  int base = 0;
  for (int i = 0; i < E; ++i) {
    const int cnt = offsets[i + 1] - offsets[i];
    const int nrb = cnt >= min_rows ? (cnt + BM - 1) / BM : 0;
    const int work = nrb * NBL;
    if (L < base + work) {
      const int li = L - base;
      const int g = li / (nrb * CG);
      const int rem = li - g * nrb * CG;
      const int gw = NBL - g * CG < CG ? NBL - g * CG : CG;
      *e = i;
      *mb = rem / gw;
      *nblock = g * CG + (rem - *mb * gw);
      return true;
    }
    base += work;
  }
  return false;
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

// Packed activations.  The grouped GEMM reads its activation operand from a
// copy laid out like the packed weights: 16-row x 32-k fragments of 1 KiB
// (lane l holds row l % 16, k = 8 (l / 16) .. +7), fragment (rb, u) at
// (rb * K/32 + u) KiB.  Each expert's dispatched rows start on a 16-row
// boundary: expert e's rows begin at packed row padded_offset(e), the rows
// past its count up to that boundary are padding.
MOE_HD inline int padded_offset(const int* offsets, int e) {
  int s = 0;
  for (int j = 0; j < e; ++j) s += (offsets[j + 1] - offsets[j] + 15) & ~15;
  return s;
}

// Upper bound on packed rows for n dispatched rows over E experts.
MOE_HD inline long long packed_rows_max(long long n, int E) { return n + 15ll * E; }

// Rows a packed buffer holds: that bound plus one 16-row block of zeros,
// which starts where the last expert's padded rows end (packed row
// padded_offset(E)).  The grouped GEMM reads it in place of the row
// fragments past an expert's last row.
MOE_HD inline long long packed_rows_alloc(long long n, int E) { return packed_rows_max(n, E) + 16; }

// Element index of (packed row prow, column k) in a packed [rows][K] matrix.
MOE_HD inline unsigned long long packed_index(long long prow, int k, int K) {
  const unsigned long long frag = (unsigned long long)(prow >> 4) * (unsigned)(K >> 5) + (unsigned)(k >> 5);
  return (frag * 64ull + (unsigned long long)((prow & 15) + 16 * ((k & 31) >> 3))) * 8ull + (unsigned)(k & 7);
}

// Byte offset of lane `lane`'s 16 bytes of packed A fragment (rb, unit 0);
// unit u adds u KiB.
MOE_HD inline unsigned long long gemm_a_offset(long long rb, int K, int lane) {
  return (unsigned long long)rb * (unsigned)(K >> 5) * 1024ull + 16ull * lane;
}

}  // namespace moe
