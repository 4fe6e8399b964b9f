// Exhaustive host check of the decode FFN launch's index arithmetic
// (moe_index.hpp, the same code the kernel runs).  Exit status 0 = pass.
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

// One launch: NG column groups x S slices x W pairs, grid padded to 8, over
// the experts whose row count lies in (min_rows, max_rows].  Returns the rows
// served per expert (from column group 0, slice 0).
static std::vector<std::vector<int>> check_launch(int NG, int W, int S, const std::vector<int>& offsets, int R,
                                                  int min_rows = 0, int max_rows = 0) {
  const int E = (int)offsets.size() - 1;
  const long long work = (long long)NG * W * S;
  const int nblk = (int)((work + 7) / 8 * 8);
  std::set<int> logical;
  std::set<std::tuple<int, int, int>> items;
  std::vector<std::vector<int>> rows_seen(E);
  for (int b = 0; b < nblk; ++b) {
    const int L = moe::xcd_logical(b, nblk);
    CHECK(L >= 0 && L < nblk, "b=%d L=%d nblk=%d", b, L, nblk);
    logical.insert(L);
    const moe::SkinnyWork w = moe::skinny_work(L, W, S);
    CHECK(w.ks >= 0 && w.ks < S && w.pair >= 0 && w.pair < W && w.ngroup >= 0, "L=%d -> (%d,%d,%d)", L, w.ngroup,
          w.ks, w.pair);
    if (w.ngroup >= NG) continue;  // padding block
    CHECK(items.insert({w.ngroup, w.ks, w.pair}).second, "duplicate item L=%d", L);
    int e, chunk, npairs;
    const bool ok = moe::skinny_pair(offsets.data(), E, R, w.pair, &e, &chunk, &npairs, min_rows, max_rows);
    CHECK(npairs <= W, "npairs %d > W %d", npairs, W);
    if (!ok) continue;
    CHECK(e >= 0 && e < E && chunk >= 0, "pair %d -> e=%d chunk=%d", w.pair, e, chunk);
    const int row0 = offsets[e] + chunk * R;
    const int nrows = std::min(R, offsets[e + 1] - row0);
    CHECK(nrows >= 1 && row0 >= offsets[e] && row0 + nrows <= offsets[e + 1], "rows [%d,+%d) outside expert %d",
          row0, nrows, e);
    // packed activations: M tile mt reads fragment row prow0/16 + min(mt, nfrag-1),
    // which must lie inside expert e's padded rows; the packed H rows written
    // are prow0 + row for row < nrows
    {
      const int pe = moe::padded_offset(offsets.data(), e);
      const int pe_end = pe + ((offsets[e + 1] - offsets[e] + 15) & ~15);
      const int prow0 = pe + chunk * R;
      const int nfrag = (nrows + 15) >> 4;
      CHECK(prow0 % 16 == 0, "skinny prow0 %d", prow0);
      for (int mt = 0; mt < R / 16; ++mt) {
        const int rb = (prow0 >> 4) + std::min(mt, nfrag - 1);
        CHECK(rb * 16 >= pe && rb * 16 + 16 <= pe_end, "skinny A fragment %d outside expert %d", rb, e);
      }
      CHECK(prow0 + nrows <= pe_end && (long long)pe_end <= moe::packed_rows_max(offsets[E], E),
            "skinny packed rows [%d,+%d) beyond expert %d end %d", prow0, nrows, e, pe_end);
    }
    if (w.ngroup == 0 && w.ks == 0)
      for (int r = row0; r < row0 + nrows; ++r) rows_seen[e].push_back(r);
  }
  CHECK((int)logical.size() == nblk, "xcd_logical not a bijection (nblk=%d)", nblk);
  CHECK((long long)items.size() == work, "items %zu != %lld", items.size(), work);
  for (int e = 0; e < E; ++e) {
    std::vector<int>& v = rows_seen[e];
    std::sort(v.begin(), v.end());
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
// pair-slot bounds; together they serve every row exactly once.
static void check_split(int N, const std::vector<int>& offsets, int hot) {
  const int E = (int)offsets.size() - 1, n = offsets[E];
  const int Wn = E + n / 64;
  const int Ww = n / 192 + n / (hot + 1) + 1;
  const auto a = check_launch(moe::skinny_groups(N, 2), Wn, 1, offsets, 64, 0, hot);
  const auto b = check_launch(moe::skinny_groups(N, 1), Ww, 1, offsets, 192, hot, 0);
  for (int e = 0; e < E; ++e)
    CHECK((int)(a[e].size() + b[e].size()) == offsets[e + 1] - offsets[e], "split: expert %d served %zu + %zu rows",
          e, a[e].size(), b[e].size());
}

// Grouped GEMM launch over packed operands: 256-row blocks, 2 x 4 waves of
// 128 x 64 (8 x 4 fragments), each wave copying A and B fragments 2w, 2w+1
// of every stage.  Checks that every copy stays inside its operand, inside its
// 32-bit offset and inside its own expert's packed rows; that the B fragment
// a wave reads is the tile and half its epilogue writes; that the packed H
// stores stay in the buffer and (when `cover`) write every output element
// exactly once; and that the row-packing kernel's reads and writes stay in
// bounds and fill every packed fragment of every expert.
static void check_gemm(int K, int N, int G, int T, int topk, const std::vector<int>& offsets, bool cover,
                       std::mt19937& rng, int min_rows = 1, int S = 1) {
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
  const long long prows = moe::packed_rows_max(n, E);
  const unsigned long long act_bytes = (unsigned long long)prows * K * 2;
  const unsigned long long h_elems = (unsigned long long)prows * N;
  const unsigned long long w_bytes = (unsigned long long)E * NB * U * G * 1024;
  const int pend = moe::padded_offset(offsets.data(), E);
  CHECK(pend % 16 == 0 && pend <= prows, "padded rows %d of %lld", pend, prows);
  std::vector<unsigned char> seen(cover ? (size_t)n * NB : 0, 0);
  std::vector<unsigned char> hwritten(cover ? (size_t)h_elems : 0, 0);
  for (int b = 0; b < nblk; ++b) {
    int e, mb, nblock;
    const int Lg = moe::xcd_logical(b, nblk);
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
        const long long rb = (prow0 >> 4) + std::min(f, nfrag - 1);
        CHECK(rb * 16 >= pe && rb * 16 + 16 <= pe_end, "A fragment %lld outside expert %d rows [%d,%d)", rb, e, pe,
              pe_end);
        for (int lane = 0; lane < 64; ++lane) {
          const unsigned long long a = moe::gemm_a_offset(rb, K, lane);
          CHECK(a < (1ull << 32) && a + (U - 1) * 1024ull + 16 <= act_bytes, "A offset %llu of %llu", a, act_bytes);
          const unsigned long long bo = moe::gemm_b_offset(e, NB, U, G, tile_base, NF, f, lane);
          CHECK(bo < (1ull << 32) && bo + (U - 1) * (unsigned long long)G * 1024 + 16 <= w_bytes,
                "B offset %llu of %llu", bo, w_bytes);
        }
      }
    for (int wm = 0; wm < WR; ++wm)
      for (int wn = 0; wn < WC; ++wn)
        for (int t = 0; t < TPW; ++t) {
          const int nb = tile_base + wn * TPW + t;
          if (nb >= NB) continue;
          for (int g = 0; g < G; ++g) {
            const unsigned long long bo = moe::gemm_b_offset(e, NB, U, G, tile_base, NF, wn * NF + t * G + g, 0);
            CHECK(bo == ((unsigned long long)(e * NB + nb) * U * G + g) * 1024ull, "B fragment of tile %d g=%d", nb,
                  g);
          }
          for (int i = 0; i < 8; ++i)
            for (int r16 = 0; r16 < 16; ++r16) {
              const int row = wm * 128 + i * 16 + r16;
              if (row >= nrows) continue;
              for (int c = 0; c < 16; ++c) {
                const unsigned long long hi = moe::packed_index(prow0 + row, nb * 16 + c, N);
                CHECK(hi < h_elems, "packed H index %llu of %llu", hi, h_elems);
                if (cover && hi < h_elems) CHECK(hwritten[hi]++ == 0, "packed H element %llu written twice", hi);
              }
              if (!cover) continue;
              unsigned char& cs = seen[(size_t)(row0 + row) * NB + nb];
              CHECK(cs == 0, "row %d tile %d written twice", row0 + row, nb);
              cs = 1;
            }
        }
  }
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
  std::vector<unsigned char> filled((size_t)(pend / 16) * U, 0);
  std::vector<int> poffs(E + 1);
  for (int i = 0; i <= E; ++i) poffs[i] = moe::padded_offset(offsets.data(), i);
  for (long long blk = 0; blk < pblocks; ++blk)
    for (int w = 0; w < 4; ++w)
      for (int lane = 0; lane < 64; ++lane) {
        const long long frag = blk * 4 + w;
        const long long rb = frag / U;
        const int u = (int)(frag - rb * U);
        const long long prow = rb * 16 + (lane & 15);
        if (prow >= pend) continue;
        int e = 0;
        while (poffs[e + 1] <= prow) ++e;
        CHECK(e < E, "pack: row %lld has no expert", prow);
        const int local = (int)(prow - poffs[e]);
        if (local < offsets[e + 1] - offsets[e]) {
          const int token = perm[offsets[e] + local] / topk;
          const unsigned long long src = (unsigned long long)token * K + u * 32 + 8 * (lane >> 4);
          CHECK(token < T && src + 8 <= (unsigned long long)T * K, "pack read %llu", src);
        }
        const unsigned long long dst = (unsigned long long)frag * 1024 + 16 * lane;
        CHECK(dst + 16 <= act_bytes, "pack write %llu of %llu", dst, act_bytes);
        if (lane == 0 && frag < (long long)filled.size()) filled[frag] = 1;
      }
  for (size_t i = 0; i < filled.size(); ++i) CHECK(filled[i], "packed fragment %zu never written", i);
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
    check_split(64 * (1 + (int)(rng() % 200)), offsets_from(counts), 64);
  }
  // grouped GEMM: the measured prefill layer (T=8192, top-2 of 8) and
  // random small shapes with ragged and empty experts
  {
    std::vector<int> counts = {2110, 1980, 2051, 2003, 2090, 2046, 2049, 2055};
    const std::vector<int> off = offsets_from(counts);
    check_gemm(4096, 14336, 2, 8192, 2, off, false, rng);
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
    check_gemm(K, N, 2, T, topk, off, true, rng);
    check_gemm(K, N, 1, T, topk, off, true, rng);
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
