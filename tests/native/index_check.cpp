// Exhaustive host check of the decode FFN launch's index arithmetic
// (moe_index.hpp, the same code the kernel runs).  Exit status 0 = pass.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <tuple>
#include <vector>

#include "moe_index.hpp"

static int fails = 0;
#define CHECK(c, ...)                         \
  do {                                        \
    if (!(c)) {                               \
      if (fails < 20) {                       \
        fprintf(stderr, "FAIL %s: ", #c);     \
        fprintf(stderr, __VA_ARGS__);         \
        fprintf(stderr, "\n");                \
      }                                       \
      ++fails;                                \
    }                                         \
  } while (0)

// The kernels number (expert, chunk) pairs with one lane per expert: lane e
// holds pair_chunks(e), the pairs before it are the prefix sum, and pair p
// belongs to the lane whose [start, start + chunks) holds it.  That must be
// skinny_pair's numbering, for every pair and the total.
static void check_pair_scan(const std::vector<int>& offsets, int R, int min_rows, int max_rows) {
  const int E = (int)offsets.size() - 1;
  std::vector<int> nch(64, 0), start(64, 0);
  int total = 0;
  for (int l = 0; l < 64; ++l) {
    nch[l] = l < E ? moe::pair_chunks(offsets.data(), l, R, min_rows, max_rows) : 0;
    start[l] = total;
    total += nch[l];
  }
  int e, chunk, np;
  moe::skinny_pair(offsets.data(), E, R, 0, &e, &chunk, &np, min_rows, max_rows);
  CHECK(total == np, "pair scan total %d != %d", total, np);
  for (int p = 0; p <= total; ++p) {
    int le = -1;
    for (int l = 0; l < 64; ++l)
      if (p >= start[l] && p < start[l] + nch[l]) {
        le = l;
        break;
      }
    const bool ok = moe::skinny_pair(offsets.data(), E, R, p, &e, &chunk, &np, min_rows, max_rows);
    CHECK(ok == (le >= 0), "pair %d: found %d vs %d", p, le >= 0, ok);
    if (ok && le >= 0) CHECK(le == e && p - start[le] == chunk, "pair %d: (%d,%d) vs (%d,%d)", p, le, p - start[le], e, chunk);
  }
}

// One kind of decode work item: NG column groups x S slices x pairs of R-row
// chunks over the experts whose row count lies in (min_rows, max_rows]; W is
// the host's upper bound on the pairs.
struct Kind {
  int NG, W, S, R, min_rows, max_rows;
};

// A decode launch of nblk blocks over kind k1, after kind k0 (the split
// launch's twelve-tile items) when given, as the kernels map blocks: the
// split launch (`real_first`) takes the pair counts derived from the offsets,
// then xcd_item and skinny_work; the one-kind launch renumbers blocks with
// xcd_logical and decodes the upper-bound grid with skinny_work, past pairs
// and column groups being padding.  Checks that every item comes out of
// exactly one block, that (real_first) on every XCD no real item follows a
// padding block in dispatch order, that each item's rows and packed fragments
// stay inside its expert, and returns the rows served per expert (from column
// group 0, slice 0).
static std::vector<std::vector<int>> check_grid(int nblk, const Kind* k0, const Kind& k1,
                                                const std::vector<int>& offsets, bool real_first) {
  const int E = (int)offsets.size() - 1;
  if (k0) check_pair_scan(offsets, k0->R, k0->min_rows, k0->max_rows);
  check_pair_scan(offsets, k1.R, k1.min_rows, k1.max_rows);
  int e, chunk, np0 = 0, np1 = 0;
  if (k0) moe::skinny_pair(offsets.data(), E, k0->R, 0, &e, &chunk, &np0, k0->min_rows, k0->max_rows);
  moe::skinny_pair(offsets.data(), E, k1.R, 0, &e, &chunk, &np1, k1.min_rows, k1.max_rows);
  CHECK(np0 <= (k0 ? k0->W : 0) && np1 <= k1.W, "pairs %d/%d above the bounds", np0, np1);
  const int n0 = k0 ? k0->NG * k0->S * np0 : 0, n1 = k1.NG * k1.S * np1;
  CHECK(nblk % 8 == 0, "grid %d", nblk);
  std::vector<int> taken(n0 + n1, 0);
  std::vector<bool> padded(8, false);
  std::vector<std::vector<int>> rows_seen(E);
  for (int b = 0; b < nblk; ++b) {
    int it;
    if (real_first) {
      it = moe::xcd_item(b, n0, n1);
    } else {
      CHECK(!k0, "the one-kind launch has no kind 0");
      const int L = moe::xcd_logical(b, nblk);
      CHECK(L >= 0 && L < nblk, "b=%d L=%d nblk=%d", b, L, nblk);
      const moe::SkinnyWork w = moe::skinny_work(L, k1.W, k1.S);
      // real items, in the numbering skinny_work(item, np1, S) decodes
      it = w.ngroup < k1.NG && w.pair < np1 ? (w.ngroup * k1.S + w.ks) * np1 + w.pair : -1;
    }
    if (it < 0) {
      padded[b & 7] = true;
      continue;
    }
    CHECK(!real_first || !padded[b & 7], "block %d: a real item after padding on XCD %d", b, b & 7);
    CHECK(it < n0 + n1, "block %d: item %d of %d", b, it, n0 + n1);
    if (it >= n0 + n1) continue;
    taken[it]++;
    const bool first = it < n0;
    const Kind& k = first ? *k0 : k1;
    const int np = first ? np0 : np1;
    const moe::SkinnyWork w = moe::skinny_work(first ? it : it - n0, np, k.S);
    CHECK(w.ngroup >= 0 && w.ngroup < k.NG && w.ks >= 0 && w.ks < k.S && w.pair >= 0 && w.pair < np,
          "item %d -> (%d,%d,%d)", it, w.ngroup, w.ks, w.pair);
    int npairs;
    const bool ok = moe::skinny_pair(offsets.data(), E, k.R, w.pair, &e, &chunk, &npairs, k.min_rows, k.max_rows);
    CHECK(ok && npairs == np, "item %d: pair %d invalid", it, w.pair);
    if (!ok) continue;
    CHECK(e >= 0 && e < E && chunk >= 0, "pair %d -> e=%d chunk=%d", w.pair, e, chunk);
    const int row0 = offsets[e] + chunk * k.R;
    const int nrows = std::min(k.R, offsets[e + 1] - row0);
    CHECK(nrows >= 1 && row0 >= offsets[e] && row0 + nrows <= offsets[e + 1], "rows [%d,+%d) outside expert %d",
          row0, nrows, e);
    // packed activations: M tile mt reads fragment row prow0/16 + min(mt, nfrag-1),
    // which must lie inside expert e's padded rows; the packed H rows written
    // are prow0 + row for row < nrows
    {
      const int pe = moe::padded_offset(offsets.data(), e);
      const int pe_end = pe + ((offsets[e + 1] - offsets[e] + 15) & ~15);
      const int prow0 = pe + chunk * k.R;
      const int nfrag = (nrows + 15) >> 4;
      CHECK(prow0 % 16 == 0, "skinny prow0 %d", prow0);
      for (int mt = 0; mt < k.R / 16; ++mt) {
        const int rb = (prow0 >> 4) + std::min(mt, nfrag - 1);
        CHECK(rb * 16 >= pe && rb * 16 + 16 <= pe_end, "skinny A fragment %d outside expert %d", rb, e);
      }
      CHECK(prow0 + nrows <= pe_end && (long long)pe_end <= moe::packed_rows_max(offsets[E], E),
            "skinny packed rows [%d,+%d) beyond expert %d end %d", prow0, nrows, e, pe_end);
    }
    if (w.ngroup == 0 && w.ks == 0)
      for (int r = row0; r < row0 + nrows; ++r) rows_seen[e].push_back(r);
  }
  for (int i = 0; i < n0 + n1; ++i) CHECK(taken[i] == 1, "item %d taken %d times (grid %d)", i, taken[i], nblk);
  for (int q = 0; q < E; ++q) std::sort(rows_seen[q].begin(), rows_seen[q].end());
  return rows_seen;
}

// One launch of one kind, grid = the host's bound rounded up to 8.  Every
// expert inside the window has each of its rows served once.
static std::vector<std::vector<int>> check_launch(int NG, int W, int S, const std::vector<int>& offsets, int R,
                                                  int min_rows = 0, int max_rows = 0) {
  const int E = (int)offsets.size() - 1;
  const long long work = (long long)NG * W * S;
  const int nblk = (int)((work + 7) / 8 * 8);
  const auto rows_seen = check_grid(nblk, nullptr, Kind{NG, W, S, R, min_rows, max_rows}, offsets, false);
  for (int e = 0; e < E; ++e) {
    const std::vector<int>& v = rows_seen[e];
    const int cnt = offsets[e + 1] - offsets[e];
    const bool in = (min_rows <= 0 || cnt > min_rows) && (max_rows <= 0 || cnt <= max_rows);
    CHECK((int)v.size() == (in ? cnt : 0), "expert %d (%d rows, window (%d,%d]) rows covered %zu", e, cnt, min_rows,
          max_rows, v.size());
    for (size_t i = 0; i < v.size(); ++i) CHECK(v[i] == offsets[e] + (int)i, "expert %d row %zu", e, i);
  }
  return rows_seen;
}

// The split decode launch: experts with at most `hot` rows in chunks of 64
// (4 M tiles), the others in chunks of 192 (12 M tiles), with the host's
// pair-slot bounds and grid (each kind's bound rounded up to 8); together
// they serve every row exactly once.
static void check_split(int N, const std::vector<int>& offsets, int hot, int ct) {
  const int E = (int)offsets.size() - 1, n = offsets[E];
  const int Wn = E + n / 64;
  const int Ww = n / 192 + n / (hot + 1) + 1;
  const Kind kw{moe::skinny_groups(N, ct), Ww, 1, 192, hot, 0}, kn{moe::skinny_groups(N, ct), Wn, 1, 64, 0, hot};
  auto round8 = [](long long v) { return (int)((v + 7) / 8 * 8); };
  const int nblk = round8((long long)kw.NG * kw.W) + round8((long long)kn.NG * kn.W);
  const auto rows = check_grid(nblk, &kw, kn, offsets, true);
  for (int e = 0; e < E; ++e) {
    CHECK((int)rows[e].size() == offsets[e + 1] - offsets[e], "split: expert %d served %zu of %d rows", e,
          rows[e].size(), offsets[e + 1] - offsets[e]);
    for (size_t i = 0; i < rows[e].size(); ++i) CHECK(rows[e][i] == offsets[e] + (int)i, "split: expert %d row %zu", e, i);
  }
}

// Grouped GEMM launch over packed operands: 256-row blocks, 2 x 4 waves of
// 128 x 64 (8 x 4 fragments), each wave copying A and B fragments 2w, 2w+1
// of every stage.  Checks that every copy stays inside its operand, inside its
// 32-bit offset and inside its own expert's packed rows; that the B fragment
// a wave reads is the tile and half its epilogue writes; that the packed H
// stores stay in the buffer and (when `cover`) write every output element
// exactly once; and that the row-packing kernel's reads and writes stay in
// bounds and fill every packed fragment of every expert.
// up = true: the up projections' placement, each XCD dealt an equal share
// of the real items (xcd_item over gemm_items), then padding; otherwise the
// grid cut into eight equal parts (xcd_logical).
static void check_gemm(int K, int N, int G, int T, int topk, const std::vector<int>& offsets, bool cover,
                       std::mt19937& rng, int min_rows = 1, int S = 1, bool up = false) {
  const int BM = 256, NF = 4, WR = 2, WC = 4, WAVES = WR * WC, CPW = 16 / WAVES, TPW = NF / G, CG = 4;
  std::set<std::tuple<int, int, int, int>> items;
  const int E = (int)offsets.size() - 1;
  const int n = offsets[E];
  const int NB = N / 16, U = K / 32;
  // the host's bound: n/256 full row blocks plus one partial per served expert
  const int W = n / BM + std::min(E, n / min_rows);
  const int tiles = WC * TPW;
  const int NBL = (NB + tiles - 1) / tiles;
  const long long work = (long long)NBL * W * S;
  const int nblk = (int)((work + 7) / 8 * 8);
  const long long prows = moe::packed_rows_alloc(n, E);
  const unsigned long long act_bytes = (unsigned long long)prows * K * 2;
  const unsigned long long h_elems = (unsigned long long)prows * N;
  const unsigned long long w_bytes = (unsigned long long)E * NB * U * G * 1024;
  const int pend = moe::padded_offset(offsets.data(), E);
  CHECK(pend % 16 == 0 && pend + 16 <= prows, "padded rows %d and the zero block of %lld", pend, prows);
  const int zrb = pend / 16;  // the zero row block
  std::vector<unsigned char> seen(cover ? (size_t)n * NB : 0, 0);
  std::vector<unsigned char> hwritten(cover ? (size_t)h_elems : 0, 0);
  CHECK(!up || (S == 1 && min_rows == 1), "up placement with S=%d min_rows=%d", S, min_rows);
  const int nreal = moe::gemm_items(offsets.data(), E, BM, NBL);
  CHECK(min_rows > 1 || nreal <= work, "gemm real items %d > grid work %lld", nreal, work);
  for (int b = 0; b < nblk; ++b) {
    int e, mb, nblock;
    const int Lg = up ? moe::xcd_item(b, nreal, 0) : moe::xcd_logical(b, nblk);
    if (Lg < 0) continue;  // padding (up placement)
    const int kslice = Lg / (NBL * W);
    if (kslice >= S) continue;
    if (!moe::gemm_item(offsets.data(), E, BM, NBL, CG, Lg - kslice * NBL * W, &e, &mb, &nblock, min_rows))
      continue;
    {
      int p0, p1;
      moe::unit_range(kslice, S, U / 2, &p0, &p1);
      CHECK(p1 > p0 && 2 * p1 <= U, "gemm slice %d of %d: units [%d,%d) of %d", kslice, S, 2 * p0, 2 * p1, U);
    }
    CHECK(offsets[e + 1] - offsets[e] >= min_rows, "expert %d with %d rows served (min %d)", e,
          offsets[e + 1] - offsets[e], min_rows);
    CHECK(items.insert({kslice, e, mb, nblock}).second, "gemm item (%d,%d,%d,%d) twice", kslice, e, mb, nblock);
    if (kslice > 0) continue;  // the rest of the checks are per item
    CHECK(e >= 0 && e < E && nblock >= 0 && nblock < NBL, "gemm item e=%d nblock=%d", e, nblock);
    const int tile_base = nblock * tiles;
    const int row0 = offsets[e] + mb * BM;
    const int nrows = std::min(BM, offsets[e + 1] - row0);
    CHECK(nrows >= 1 && row0 + nrows <= offsets[e + 1], "gemm rows [%d,+%d) e=%d", row0, nrows, e);
    const int pe = moe::padded_offset(offsets.data(), e);
    const int pe_end = pe + ((offsets[e + 1] - offsets[e] + 15) & ~15);
    const int prow0 = pe + mb * BM;
    const int nfrag = (nrows + 15) >> 4;
    CHECK(prow0 % 16 == 0, "prow0 %d", prow0);
    for (int wave = 0; wave < WAVES; ++wave)
      for (int j = 0; j < CPW; ++j) {
        const int f = CPW * wave + j;
        CHECK(16 + f < 32, "lds slot %d", 16 + f);
        // fragments past the expert's last row read the zero row block
        const long long rb = f < nfrag ? (prow0 >> 4) + f : zrb;
        CHECK(rb == zrb || (rb * 16 >= pe && rb * 16 + 16 <= pe_end), "A fragment %lld outside expert %d rows [%d,%d)",
              rb, e, pe, pe_end);
        for (int lane = 0; lane < 64; ++lane) {
          const unsigned long long a = moe::gemm_a_offset(rb, K, lane);
          CHECK(a < (1ull << 32) && a + (U - 1) * 1024ull + 16 <= act_bytes, "A offset %llu of %llu", a, act_bytes);
          const unsigned long long bo = moe::gemm_b_offset(e, NB, U, G, tile_base, NF, f, lane);
          CHECK(bo < (1ull << 32) && bo + (U - 1) * (unsigned long long)G * 1024 + 16 <= w_bytes,
                "B offset %llu of %llu", bo, w_bytes);
        }
      }
    for (int wm = 0; wm < WR; ++wm)
      for (int wn = 0; wn < WC; ++wn) {
        // the epilogue: a wave's TPW tiles are KF whole 32-column packed
        // fragments of each of its 8 row fragments; the fragments that start
        // before the block's last real row are copied out whole (their
        // padding rows included), the others not at all
        const int nb0 = tile_base + wn * TPW;
        CHECK(NB % 4 == 0 && nb0 % TPW == 0, "wave tiles %d.. of %d", nb0, NB);
        if (nb0 >= NB) continue;
        CHECK(nb0 + TPW <= NB && (nb0 * 16) % 32 == 0, "wave columns %d..+%d of %d", nb0 * 16, TPW * 16, N);
        const int KF = TPW / 2;
        // the first row block of the first expert served also zeroes H's
        // zero row block (wave row 0, the wave's own fragments)
        if (mb == 0 && offsets[e] == 0 && wm == 0)
          for (int kf = 0; kf < KF; ++kf) {
            const unsigned long long frag = (unsigned long long)zrb * (N >> 5) + (nb0 >> 1) + kf;
            for (int x = 0; x < 512; ++x) {
              const unsigned long long hi = frag * 512 + x;
              CHECK(hi < h_elems, "zero H index %llu of %llu", hi, h_elems);
              if (cover && hi < h_elems) CHECK(hwritten[hi]++ == 0, "zero H element %llu written twice", hi);
            }
          }
        for (int i = 0; i < 8; ++i) {
          if (wm * 128 + 16 * i >= nrows) break;
          const int fprow = prow0 + wm * 128 + 16 * i;
          CHECK(fprow >= pe && fprow + 16 <= pe_end, "H fragment rows [%d,+16) outside expert %d [%d,%d)", fprow, e, pe,
                pe_end);
          for (int kf = 0; kf < KF; ++kf) {
            const unsigned long long frag = (unsigned long long)(fprow >> 4) * (N >> 5) + (nb0 >> 1) + kf;
            CHECK(frag == moe::packed_index(fprow, nb0 * 16 + 32 * kf, N) / 512, "H fragment %llu", frag);
            for (int x = 0; x < 512; ++x) {
              const unsigned long long hi = frag * 512 + x;
              CHECK(hi < h_elems, "packed H index %llu of %llu", hi, h_elems);
              if (cover && hi < h_elems) CHECK(hwritten[hi]++ == 0, "packed H element %llu written twice", hi);
            }
          }
        }
        for (int t = 0; t < TPW; ++t) {
          const int nb = nb0 + t;
          for (int g = 0; g < G; ++g) {
            const unsigned long long bo = moe::gemm_b_offset(e, NB, U, G, tile_base, NF, wn * NF + t * G + g, 0);
            CHECK(bo == ((unsigned long long)(e * NB + nb) * U * G + g) * 1024ull, "B fragment of tile %d g=%d", nb,
                  g);
          }
          for (int i = 0; i < 8; ++i)
            for (int r16 = 0; r16 < 16; ++r16) {
              const int row = wm * 128 + i * 16 + r16;
              if (row >= nrows) continue;
              if (cover) {  // every real row's element is inside a copied fragment
                const unsigned long long hi = moe::packed_index(prow0 + row, nb * 16, N);
                CHECK(hi < h_elems && hwritten[hi] == 1, "real H element %llu not written", hi);
              }
              if (!cover) continue;
              unsigned char& cs = seen[(size_t)(row0 + row) * NB + nb];
              CHECK(cs == 0, "row %d tile %d written twice", row0 + row, nb);
              cs = 1;
            }
        }
      }
  }
  if (cover && n > 0 && min_rows == 1)  // H's zero row block: every fragment written once
    for (unsigned long long hi = (unsigned long long)zrb * 16 * N; hi < (unsigned long long)(zrb + 1) * 16 * N; ++hi)
      CHECK(hwritten[hi] == 1, "zero H element %llu written %d times", hi, (int)hwritten[hi]);
  long long nitems = 0;
  for (int i = 0; i < E; ++i)
    if (offsets[i + 1] - offsets[i] >= min_rows) nitems += (long long)((offsets[i + 1] - offsets[i] + BM - 1) / BM) * NBL;
  CHECK((long long)items.size() == nitems * S, "gemm items %zu of %lld x %d", items.size(), nitems, S);
  CHECK(nitems * S <= work, "gemm items %lld > grid work %lld", nitems * S, work);
  if (cover)
    for (size_t i = 0; i < seen.size(); ++i) {
      int ei = 0;
      while (offsets[ei + 1] <= (int)(i / NB)) ++ei;
      const bool served = offsets[ei + 1] - offsets[ei] >= min_rows;
      CHECK(seen[i] == (served ? 1 : 0), "row %zu tile %zu written %d times", i / NB, i % NB, (int)seen[i]);
    }
  // the row-packing kernel: 4 waves per block, one fragment per wave
  if (!cover) return;
  std::vector<int> perm(n);
  for (int i = 0; i < n; ++i) perm[i] = (int)(rng() % std::max(1, T * topk));
  const long long frags = prows / 16 * U;
  const long long pblocks = (frags + 3) / 4;
  std::vector<unsigned char> filled((size_t)(pend / 16 + 1) * U, 0);  // the zero row block included
  std::vector<int> poffs(E + 1);
  for (int i = 0; i <= E; ++i) poffs[i] = moe::padded_offset(offsets.data(), i);
  for (long long blk = 0; blk < pblocks; ++blk)
    for (int w = 0; w < 4; ++w)
      for (int lane = 0; lane < 64; ++lane) {
        const long long frag = blk * 4 + w;
        const long long rb = frag / U;
        const int u = (int)(frag - rb * U);
        const long long prow = rb * 16 + (lane & 15);
        if (prow >= pend + 16) continue;
        int e = 0;
        if (prow < pend)
          while (poffs[e + 1] <= prow) ++e;
        CHECK(e < E, "pack: row %lld has no expert", prow);
        const int local = (int)(prow - poffs[e]);
        if (prow < pend && local < offsets[e + 1] - offsets[e]) {
          const int token = perm[offsets[e] + local] / topk;
          const unsigned long long src = (unsigned long long)token * K + u * 32 + 8 * (lane >> 4);
          CHECK(token < T && src + 8 <= (unsigned long long)T * K, "pack read %llu", src);
        }
        const unsigned long long dst = (unsigned long long)frag * 1024 + 16 * lane;
        CHECK(dst + 16 <= act_bytes, "pack write %llu of %llu", dst, act_bytes);
        if (lane == 0 && frag < (long long)filled.size()) filled[frag] = 1;
      }
  for (size_t i = 0; i < filled.size(); ++i) CHECK(filled[i], "packed fragment %zu never written", i);
  // the four-fragment packing kernel (dispatch given, K / 32 a multiple of 4):
  // a wave writes fragments 4 w' .. 4 w' + 3 of one 16-row block, each lane
  // reading 16 bytes of its row at k = u0 * 32 + 8 (lane / 16) + 32 f
  if (U % 4) return;
  std::fill(filled.begin(), filled.end(), 0);
  const long long pblocks4 = (frags / 4 + 3) / 4;
  for (long long blk = 0; blk < pblocks4; ++blk)
    for (int w = 0; w < 4; ++w)
      for (int lane = 0; lane < 64; ++lane) {
        const long long frag0 = (blk * 4 + w) * 4;
        const long long rb = frag0 / U;
        const int u0 = (int)(frag0 - rb * U);
        CHECK(u0 + 3 < U, "pack4: fragments %lld..+3 cross a row block", frag0);
        const long long prow = rb * 16 + (lane & 15);
        if (prow >= pend + 16) continue;
        int e = 0;
        if (prow < pend)
          while (poffs[e + 1] <= prow) ++e;
        CHECK(e < E, "pack4: row %lld has no expert", prow);
        const int local = (int)(prow - poffs[e]);
        for (int f = 0; f < 4; ++f) {
          if (prow < pend && local < offsets[e + 1] - offsets[e]) {
            const int token = perm[offsets[e] + local] / topk;
            const unsigned long long src = (unsigned long long)token * K + u0 * 32 + 8 * (lane >> 4) + 32 * f;
            CHECK(token < T && src + 8 <= (unsigned long long)T * K, "pack4 read %llu", src);
            CHECK(src / K == (unsigned long long)token, "pack4 read %llu leaves row %d", src, token);
          }
          const unsigned long long dst = (unsigned long long)(frag0 + f) * 1024 + 16 * lane;
          CHECK(dst + 16 <= act_bytes, "pack4 write %llu of %llu", dst, act_bytes);
          if (lane == 0 && frag0 + f < (long long)filled.size()) filled[frag0 + f] += 1;
        }
      }
  for (size_t i = 0; i < filled.size(); ++i) CHECK(filled[i] == 1, "pack4: packed fragment %zu written %d times", i,
                                                   (int)filled[i]);
}

// Decode FFN column groups: every 16-column tile is owned by exactly one
// (group, wave), and no wave owns tiles on both sides of N/16.
static void check_skinny_tiles(int N, int CT) {
  const int NB = N / 16, NG = moe::skinny_groups(N, CT);
  std::vector<int> owned(NB, 0);
  for (int g = 0; g < NG; ++g)
    for (int w = 0; w < 4; ++w) {
      const int t0 = (g * 4 + w) * CT;
      int in = 0;
      for (int c = 0; c < CT; ++c)
        if (t0 + c < NB) {
          ++owned[t0 + c];
          ++in;
        }
      CHECK(in == 0 || in == CT, "N=%d CT=%d group %d wave %d owns %d of %d tiles", N, CT, g, w, in, CT);
    }
  for (int t = 0; t < NB; ++t) CHECK(owned[t] == 1, "N=%d CT=%d tile %d owned %d times", N, CT, t, owned[t]);
}

static void check_units(int U, int parts) {
  int prev = 0;
  for (int p = 0; p < parts; ++p) {
    int u0, u1;
    moe::unit_range(p, parts, U, &u0, &u1);
    CHECK(u0 == prev && u1 >= u0 && u1 <= U, "U=%d parts=%d p=%d [%d,%d)", U, parts, p, u0, u1);
    prev = u1;
  }
  CHECK(prev == U, "U=%d parts=%d ends at %d", U, parts, prev);
}

static std::vector<int> offsets_from(const std::vector<int>& counts) {
  std::vector<int> o(counts.size() + 1, 0);
  for (size_t i = 0; i < counts.size(); ++i) o[i + 1] = o[i] + counts[i];
  return o;
}

int main() {
  std::mt19937 rng(1234);
  // the measured layers' shapes, with their realised or typical counts
  struct Case {
    int N, E, n, R, CT, S;
    std::vector<int> counts;
  };
  std::vector<Case> cases = {
      {14336, 8, 32, 16, 1, 1, {5, 8, 3, 3, 4, 4, 4, 1}},
      {4096, 8, 32, 16, 1, 4, {5, 8, 3, 3, 4, 4, 4, 1}},
      {6400, 16, 512, 64, 2, 1, {165, 106, 61, 38, 36, 22, 19, 12, 11, 8, 9, 3, 11, 3, 5, 3}},
      {4096, 16, 512, 64, 2, 4, {165, 106, 61, 38, 36, 22, 19, 12, 11, 8, 9, 3, 11, 3, 5, 3}},
      {14336, 8, 128, 32, 4, 1, {20, 11, 15, 16, 22, 16, 15, 13}},
      {4096, 8, 128, 32, 4, 4, {20, 11, 15, 16, 22, 16, 15, 13}},
  };
  for (auto& c : cases) {
    const int W = c.E + c.n / c.R;
    check_launch(moe::skinny_groups(c.N, c.CT), W, c.S, offsets_from(c.counts), c.R);  // waves split columns
    check_launch(c.N / 16 / c.CT, W, c.S, offsets_from(c.counts), c.R);                 // waves split K
  }
  // random shapes, including empty experts and one expert holding everything
  for (int it = 0; it < 300; ++it) {
    const int E = 1 + (int)(rng() % 64);
    const int R = 16 << (rng() % 3);
    const int CT = 1 << (rng() % 3);
    const int S = 1 + (int)(rng() % 4);
    const int NB = 4 * (1 + (int)(rng() % 64));
    const int n = (int)(rng() % 3000);
    std::vector<int> counts(E, 0);
    const int mode = it % 3;
    for (int a = 0; a < n; ++a) counts[mode == 0 ? (int)(rng() % E) : (mode == 1 ? 0 : (int)(rng() % (1 + E / 4)))]++;
    const int W = E + n / R;
    check_launch(moe::skinny_groups(NB * 16, CT), W, S, offsets_from(counts), R);
    check_launch(NB / CT, W, S, offsets_from(counts), R);
  }
  // split decode launch: Zipf-like skews with one to a few hot experts
  for (int it = 0; it < 300; ++it) {
    const int E = 1 + (int)(rng() % 64);
    const int n = (int)(rng() % 2500);
    std::vector<int> counts(E, 0);
    for (int a = 0; a < n; ++a) {
      const double r = std::uniform_real_distribution<double>(0.0, 1.0)(rng);
      counts[std::min(E - 1, (int)(E * r * r * r))]++;
    }
    check_split(64 * (1 + (int)(rng() % 200)), offsets_from(counts), 64, 1 + (int)(rng() % 2));
  }
  // grouped GEMM: the measured prefill layer (T=8192, top-2 of 8) and
  // random small shapes with ragged and empty experts
  {
    std::vector<int> counts = {2110, 1980, 2051, 2003, 2090, 2046, 2049, 2055};
    const std::vector<int> off = offsets_from(counts);
    check_gemm(4096, 14336, 2, 8192, 2, off, false, rng, 1, 1, true);
    check_gemm(14336, 4096, 1, 8192, 2, off, false, rng);
  }
  for (int it = 0; it < 120; ++it) {
    const int E = 1 + (int)(rng() % 16);
    const int topk = 1 + (int)(rng() % std::min(E, 4));
    const int T = (int)(rng() % 1500);
    const int K = 64 * (1 + (int)(rng() % 12));
    const int N = 64 * (1 + (int)(rng() % 12));
    std::vector<int> counts(E, 0);
    for (int a = 0; a < T * topk; ++a) counts[it % 2 ? (int)(rng() % E) : (int)(rng() % (1 + E / 3))]++;
    const std::vector<int> off = offsets_from(counts);
    check_gemm(K, N, 2, T, topk, off, true, rng, 1, 1, true);
    check_gemm(K, N, 1, T, topk, off, true, rng, 1, 1, true);
    check_gemm(N, K, 1, T, topk, off, true, rng);
    const int hot = 1 + (int)(rng() % 130);  // the hybrid split: experts with >= hot rows
    check_gemm(K, N, 2, T, topk, off, true, rng, hot);
    check_gemm(N, K, 1, T, topk, off, true, rng, hot);
    check_gemm(N, K, 1, T, topk, off, true, rng, hot, 1 + (int)(rng() % std::min(8, N / 64)));
  }
  for (int N = 64; N <= 14336 * 2; N += 64)
    for (int CT : {1, 2, 4}) check_skinny_tiles(N, CT);
  for (int U : {1, 2, 7, 50, 112, 128, 200, 448})
    for (int parts : {1, 4, 8, 16, 32}) check_units(U, parts);
  if (fails) {
    fprintf(stderr, "%d failures\n", fails);
    return 1;
  }
  printf("index check ok\n");
  return 0;
}
