// Host build of the attention kernel's chip schedule (attn_sched.h, the same
// source the kernels include), checked exhaustively over shape sweeps:
//  - xcd_order is a bijection of [0, n);
//  - spread_tile is a bijection of [0, nq * nbh) onto (rank, head);
//  - win_span covers every key any row of a query tile can see, reads no
//    sub-tile past the valid keys, and claims `fast` only when every row of
//    the tile sees the same whole sub-tiles (brute force over frames);
//  - win_rank_key ranks query blocks as a permutation, longest first;
//  - the split of the last partial round: every split block's steps and
//    records, the coverage of every split tile's steps exactly once, the
//    merge's inverse map, and every record index below the slots reserved.
// Prints "WS B Sq Sk H D part_slots max_record" for the workload shapes so
// the Python side can compare with the library's workspace size; exits 1 on
// the first failure, printing it.
#define __host__
#define __device__
#include "attn_sched.h"

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

using namespace h3;

static long long g_checks = 0;

#define REQUIRE(cond, ...)                                   \
  do {                                                       \
    ++g_checks;                                              \
    if (!(cond)) {                                           \
      std::fprintf(stderr, "FAIL %s:%d: %s | ", __FILE__, __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                     \
      std::fprintf(stderr, "\n");                            \
      std::exit(1);                                          \
    }                                                        \
  } while (0)

static void check_xcd_order() {
  for (int n = 0; n <= 5000; ++n) {
    std::vector<char> seen(n, 0);
    for (int i = 0; i < n; ++i) {
      const int g = xcd_order(i, n);
      REQUIRE(g >= 0 && g < n && !seen[g], "n=%d i=%d g=%d", n, i, g);
      seen[g] = 1;
    }
  }
}

static void check_spread(int nq, int nbh, bool ragged) {
  std::vector<char> seen((size_t)nq * nbh, 0);
  for (int bid = 0; bid < nq * nbh; ++bid) {
    int rank = -1, bh = -1;
    spread_tile(bid, nq, nbh, ragged, rank, bh);
    REQUIRE(rank >= 0 && rank < nq && bh >= 0 && bh < nbh, "nq=%d nbh=%d ragged=%d bid=%d -> (%d,%d)", nq, nbh,
            (int)ragged, bid, rank, bh);
    char& s = seen[(size_t)rank * nbh + bh];
    REQUIRE(!s, "nq=%d nbh=%d ragged=%d bid=%d -> (%d,%d) twice", nq, nbh, (int)ragged, bid, rank, bh);
    s = 1;
  }
}

static void check_spread_tile() {
  for (int nq = 1; nq <= 80; ++nq)
    for (int nbh = 1; nbh <= 60; ++nbh)
      for (int rg = 0; rg < 2; ++rg) check_spread(nq, nbh, rg != 0);
  // Workload geometries: full (408 x 6), head dim 64 (408 x 12) and 256
  // (816 x 3), padded (128 x 8), cross (128 x 8), mid (32 x 8), per-item
  // lengths (128 x 32), and a few wide ones.
  const int shapes[][2] = {{408, 6}, {408, 12}, {816, 3}, {128, 8}, {32, 8}, {128, 32}, {408, 48},
                           {1024, 5}, {1000, 96}, {3, 1000}, {817, 7}};
  for (const auto& s : shapes)
    for (int rg = 0; rg < 2; ++rg) check_spread(s[0], s[1], rg != 0);
}

// Frame visibility written from its definition, independent of win_span.
static bool visible(int i, int j, int F, int C, int R, int A) {
  const int fi = i / F, fj = j / F;
  if (fi < A || fj < A) return true;
  const int ci = (fi - A) / C, cj = (fj - A) / C;
  return ci - cj <= R && cj - ci <= R;
}

static void check_win_tile(int F, int C, int R, int A, int BM, int q00, int qv, int kvv) {
  const WinSpan w = win_span(F, C, R, A, BM, q00, qv, kvv);
  const int NU = (kvv + kAttnSub - 1) / kAttnSub;
  REQUIRE(w.wn1 >= 0 && w.ws2 >= 0 && w.xe >= w.wn1, "F=%d C=%d R=%d A=%d q00=%d kvv=%d: wn1=%d ws2=%d xe=%d", F, C,
          R, A, q00, kvv, w.wn1, w.ws2, w.xe);
  REQUIRE(w.xe == w.wn1 || w.ws2 >= 0, "range order");
  // Sub-tiles the kernel walks.
  std::vector<char> walked(NU, 0);
  for (int v = 0; v < w.xe; ++v) {
    const int x = v < w.wn1 ? v : v + w.ws2;
    REQUIRE(x >= 0 && x < NU, "F=%d C=%d R=%d A=%d q00=%d kvv=%d: step %d reads sub-tile %d of %d", F, C, R, A, q00,
            kvv, v, x, NU);
    REQUIRE(!walked[x], "sub-tile %d walked twice", x);
    walked[x] = 1;
  }
  // Visible keys per distinct row frame (visibility depends on frames only).
  const int q1 = std::min(q00 + BM, qv);
  std::vector<char> first_set;
  bool same = true;
  for (int f = q00 / F; f <= (q1 - 1) / F; ++f) {
    const int i = std::max(f * F, q00);
    std::vector<char> vis(kvv, 0);
    for (int fj = 0; fj * F < kvv; ++fj) {
      const bool s = visible(i, fj * F, F, C, R, A);
      for (int j = fj * F; j < std::min((fj + 1) * F, kvv); ++j) vis[j] = s;
    }
    for (int j = 0; j < kvv; ++j)
      REQUIRE(!vis[j] || walked[j / kAttnSub], "F=%d C=%d R=%d A=%d BM=%d q00=%d qv=%d kvv=%d: key %d of row %d not walked",
              F, C, R, A, BM, q00, qv, kvv, j, i);
    if (first_set.empty()) first_set = vis;
    else if (vis != first_set) same = false;
  }
  if (w.fast) {
    REQUIRE(same, "F=%d C=%d R=%d A=%d q00=%d: fast tile whose rows see different keys", F, C, R, A, q00);
    for (int j = 0; j < kvv; ++j)
      REQUIRE(first_set[j] == walked[j / kAttnSub], "F=%d C=%d R=%d A=%d BM=%d q00=%d kvv=%d: fast tile, key %d %s", F,
              C, R, A, BM, q00, kvv, j, first_set[j] ? "visible but not walked" : "walked but hidden");
  }
}

static void check_win_span() {
  const int Fs[] = {1, 7, 32, 33, 100, 256, 300, 1024, 3072};
  const int Ss[] = {1, 31, 257, 1000, 3072};
  for (int F : Fs)
    for (int C = 1; C <= 5; C += 2)
      for (int R = 0; R <= 2; ++R)
        for (int A = 0; A <= 2; ++A)
          for (int S : Ss)
            for (int BM : {128, 256})
              for (int kvv : {S, (S + 1) / 2, 1})
                for (int qv : {S, (2 * S + 2) / 3})
                  for (int q00 = 0; q00 < qv; q00 += BM) check_win_tile(F, C, R, A, BM, q00, qv, kvv);
  // The full_window geometry: 34 frames of 3072 rows, chunks of 5, radius 1,
  // one anchor frame, 104448 rows.
  for (int q00 = 0; q00 < 104448; q00 += 256) check_win_tile(3072, 5, 1, 1, 256, q00, 104448, 104448);
}

static void check_rank_keys() {
  uint32_t lcg = 12345u;
  for (int n = 1; n <= kWinOrderMax; n = n < 64 ? n + 1 : n * 2 - 1) {
    if (n > kWinOrderMax) break;
    std::vector<int> xe(n);
    for (int j = 0; j < n; ++j) {
      lcg = lcg * 1664525u + 1013904223u;
      xe[j] = (j % 3 == 0) ? (int)(lcg >> 28) : (int)(lcg >> 10);   // many ties, and spans up to 2^22
    }
    std::vector<uint32_t> key(n);
    for (int j = 0; j < n; ++j) key[j] = win_rank_key(xe[j], j);
    std::vector<int> block_of_rank(n, -1);
    for (int j = 0; j < n; ++j) {
      REQUIRE(key[j] > 0, "padding key");
      int r = 0;
      for (int i = 0; i < n; ++i) r += key[i] > key[j] ? 1 : 0;
      REQUIRE(block_of_rank[r] < 0, "n=%d rank %d twice", n, r);
      block_of_rank[r] = j;
    }
    for (int r = 1; r < n; ++r) {
      const int a = block_of_rank[r - 1], b = block_of_rank[r];
      const int xa = std::min(xe[a], (1 << 21) - 1), xb = std::min(xe[b], (1 << 21) - 1);
      REQUIRE(xa > xb || (xa == xb && a < b), "n=%d: rank %d block %d before block %d", n, r, a, b);
    }
  }
}

struct Shape {
  int B, Sq, Sk, H, qv, kvv;
};

static int64_t check_split(const Shape& s, int D, int QT, int cus) {
  const int BM = attn_rows(D, QT);
  const int64_t part_slots = split_part_slots(s.B, s.Sq, s.Sk, s.H, D);
  const int64_t nqv = (s.qv + BM - 1) / BM;
  const int64_t n_valid = (int64_t)s.B * s.H * nqv;
  const int NU = (s.kvv + kAttnSub - 1) / kAttnSub;
  const SplitPlan p = split_plan(n_valid, NU, cus, part_slots);
  REQUIRE(p.n_whole + p.n_split == n_valid, "tiles");
  int64_t max_rec = -1;
  if (p.n_split == 0) {
    REQUIRE(p.n_blocks == 0 && p.n_whole == n_valid, "no split");
    return max_rec;
  }
  const int nsp = (int)p.n_split, nb = (int)p.n_blocks;
  REQUIRE(nb > nsp && nb <= std::min(cus, kSplitMaxBlocks) && nb <= part_slots / 2,
          "B=%d Sq=%d Sk=%d H=%d D=%d cus=%d: %d blocks for %d tiles, %lld slots", s.B, s.Sq, s.Sk, s.H, D, cus, nb,
          nsp, (long long)part_slots);
  REQUIRE(p.n_whole % std::min(cus, kSplitMaxBlocks) == 0, "whole rounds");
  const int64_t U = (int64_t)nsp * NU;
  std::vector<SplitSeg> seg(nb);
  std::vector<char> seen(nb, 0);
  for (int b = 0; b < nb; ++b) {
    const int j = xcd_order(b, nb);
    REQUIRE(j >= 0 && j < nb && !seen[j], "xcd_order over split blocks");
    seen[j] = 1;
  }
  std::vector<int> steps(nsp, 0);
  int64_t next = 0;
  for (int j = 0; j < nb; ++j) {
    const SplitSeg g = split_segments(j, nsp, NU, nb);
    seg[j] = g;
    const int64_t s0 = (int64_t)g.tile * NU + g.xb0;
    REQUIRE(s0 == next, "B=%d Sq=%d Sk=%d H=%d D=%d cus=%d block %d starts at %lld, expected %lld", s.B, s.Sq, s.Sk,
            s.H, D, cus, j, (long long)s0, (long long)next);
    REQUIRE(g.tile >= 0 && g.tile < nsp && g.xb0 >= 0 && g.xb0 < g.xe0 && g.xe0 <= NU, "segment 0 of block %d", j);
    REQUIRE(g.rec0 == 2 * j && g.rec0 < part_slots, "record %d of %lld", g.rec0, (long long)part_slots);
    max_rec = std::max<int64_t>(max_rec, g.rec0);
    steps[g.tile] += g.xe0 - g.xb0;
    next = (int64_t)g.tile * NU + g.xe0;
    if (g.nseg == 2) {
      REQUIRE(g.xe0 == NU && g.tile + 1 < nsp && g.xe1 > 0 && g.xe1 <= NU, "segment 1 of block %d", j);
      REQUIRE(g.rec1 == 2 * j + 1 && g.rec1 < part_slots, "record %d of %lld", g.rec1, (long long)part_slots);
      max_rec = std::max<int64_t>(max_rec, g.rec1);
      steps[g.tile + 1] += g.xe1;
      next = (int64_t)(g.tile + 1) * NU + g.xe1;
    } else {
      REQUIRE(g.nseg == 1 && g.rec1 == -1, "one segment");
    }
  }
  REQUIRE(next == U, "blocks cover %lld of %lld steps", (long long)next, (long long)U);
  // The key sub-tiles each block reads: every split tile's [0, NU) exactly
  // once, each segment a range inside [0, NU), and a block that starts in a
  // tile as the first there begins at key sub-tile 0.
  std::vector<std::vector<uint8_t>> keys(nsp, std::vector<uint8_t>(NU, 0));
  for (int j = 0; j < nb; ++j) {
    const SplitSeg& g = seg[j];
    const int n0 = g.xe0 - g.xb0;
    REQUIRE(g.kb0 >= 0 && g.kb0 + n0 <= NU, "block %d keys [%d, %d) of %d", j, g.kb0, g.kb0 + n0, NU);
    for (int x = g.kb0; x < g.kb0 + n0; ++x) keys[g.tile][x]++;
    if (j == 0 || seg[j - 1].tile < g.tile)   // the first block that starts inside its tile
      REQUIRE(g.kb0 == 0, "first block %d of tile %d starts at key sub-tile %d", j, g.tile, g.kb0);
    if (g.nseg == 2) {
      REQUIRE(g.kb1 >= 0 && g.kb1 + g.xe1 == NU, "block %d second keys [%d, %d) of %d", j, g.kb1, g.kb1 + g.xe1, NU);
      for (int x = g.kb1; x < g.kb1 + g.xe1; ++x) keys[g.tile + 1][x]++;
    }
  }
  for (int t = 0; t < nsp; ++t)
    for (int x = 0; x < NU; ++x)
      REQUIRE(keys[t][x] == 1, "tile %d key sub-tile %d read %d times", t, x, (int)keys[t][x]);
  for (int t = 0; t < nsp; ++t) {
    REQUIRE(steps[t] == NU, "tile %d covered %d of %d steps", t, steps[t], NU);
    int j0, j1;
    merge_blocks(t, nsp, NU, nb, j0, j1);
    REQUIRE(j0 >= 0 && j0 <= j1 && j1 < nb, "merge range of tile %d: %d..%d", t, j0, j1);
    int covered = 0;
    for (int j = 0; j < nb; ++j) {
      const SplitSeg& g = seg[j];
      int rec = -1, n = 0;
      if (g.tile == t) { rec = g.rec0; n = g.xe0 - g.xb0; }
      else if (g.nseg == 2 && g.tile + 1 == t) { rec = g.rec1; n = g.xe1; }
      const bool in = j >= j0 && j <= j1;
      REQUIRE(in == (rec >= 0), "tile %d: block %d %s the merge range %d..%d", t, j, in ? "in" : "outside", j0, j1);
      if (in) {
        REQUIRE(merge_record(j, t, nsp, NU, nb) == rec, "tile %d block %d: merge reads record %d, block wrote %d", t, j,
                merge_record(j, t, nsp, NU, nb), rec);
        covered += n;
      }
    }
    REQUIRE(covered == NU, "merge of tile %d sees %d of %d steps", t, covered, NU);
  }
  return max_rec;
}

int main() {
  check_xcd_order();
  check_spread_tile();
  check_win_span();
  check_rank_keys();

  // The workloads' shapes (tiny, mid, padded, cross, full; the head-dim 64
  // and 256 full sequences), then seeded random ones.
  std::vector<std::pair<Shape, int>> shapes = {
      {{1, 512, 512, 2, 512, 512}, 128},         {{1, 8192, 8192, 8, 8192, 8192}, 128},
      {{1, 32768, 32768, 8, 30720, 30720}, 128}, {{1, 32760, 512, 8, 32760, 300}, 128},
      {{1, 104448, 104448, 6, 104448, 104448}, 128}, {{1, 104448, 104448, 12, 104448, 104448}, 64},
      {{1, 104448, 104448, 3, 104448, 104448}, 256}, {{1, 104448, 104448, 6, 104448, 104448}, 64},
      {{1, 104448, 104448, 6, 104448, 104448}, 256}, {{2, 4000, 3500, 2, 3500, 3333}, 128},
      {{1, 3000, 3000, 3, 3000, 3000}, 128},     {{1, 2100, 1200, 1, 2100, 1100}, 128},
      {{1, 16640, 16640, 4, 16640, 16640}, 128}, {{4, 32768, 32768, 8, 32768, 32768}, 128},
  };
  const int n_fixed = (int)shapes.size();
  uint64_t st = 0x9E3779B97F4A7C15ull;
  auto rnd = [&](int lo, int hi) {
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return lo + (int)(st % (uint64_t)(hi - lo + 1));
  };
  for (int i = 0; i < 4000; ++i) {
    Shape s;
    s.B = rnd(1, 4);
    s.H = rnd(1, 16);
    s.Sq = rnd(1, i % 4 == 0 ? 60000 : 9000);
    s.Sk = rnd(1, i % 5 == 0 ? 60000 : 9000);
    s.qv = rnd(0, s.Sq);
    s.kvv = rnd(1, s.Sk);
    const int D = (i % 3 == 0) ? 64 : (i % 3 == 1 ? 128 : 256);
    shapes.push_back({s, D});
  }
  const int cus_list[] = {1, 7, 8, 33, 64, 80, 104, 120, 128, 200, 255, 256, 257, 304, 1024};
  int n_split_cases = 0;
  for (size_t i = 0; i < shapes.size(); ++i) {
    int64_t max_rec = -1;
    const int D = shapes[i].second;
    const Shape& s = shapes[i].first;
    for (int cus : cus_list) {
      for (int QT = attn_qt_min(D); QT <= attn_qt_max(D); ++QT) {
        const int64_t m = check_split(s, D, QT, cus);
        if (m >= 0) ++n_split_cases;
        max_rec = std::max(max_rec, m);
      }
      // The launcher's choice is one of the head dim's tilings in both modes.
      const int64_t NU = (s.kvv + kAttnSub - 1) / kAttnSub;
      const int64_t slots = split_part_slots(s.B, s.Sq, s.Sk, s.H, D);
      for (int general = 0; general < 2; ++general) {
        const int qt = choose_query_tiles(D, general != 0, (int64_t)s.B * s.H, general ? s.Sq : s.qv, NU, cus, slots);
        REQUIRE(qt >= attn_qt_min(D) && qt <= attn_qt_max(D), "D=%d: %d query tiles", D, qt);
      }
    }
    if ((int)i < n_fixed) {
      std::printf("WS %d %d %d %d %d %lld %lld\n", s.B, s.Sq, s.Sk, s.H, D,
                  (long long)split_part_slots(s.B, s.Sq, s.Sk, s.H, D), (long long)max_rec);
      const int64_t NU = (s.kvv + kAttnSub - 1) / kAttnSub;
      std::printf("QT %d %d %d %d %d %d %d %d\n", s.B, s.Sq, s.Sk, s.H, D, s.qv, s.kvv,
                  choose_query_tiles(D, false, (int64_t)s.B * s.H, s.qv, NU, 256,
                                     split_part_slots(s.B, s.Sq, s.Sk, s.H, D)));
    }
  }
  std::printf("OK %lld checks, %zu split shapes x %zu CU counts (%d split)\n", g_checks, shapes.size(),
              sizeof(cus_list) / sizeof(cus_list[0]), n_split_cases);
  return 0;
}
