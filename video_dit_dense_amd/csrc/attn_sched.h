// Chip schedule of the attention kernel: the tile orders and the split of the
// last partial round of tiles, as plain integer arithmetic that the kernels,
// the launcher and a host-compiled check all include. Nothing here touches
// memory or depends on HIP; a host build defines __host__ and __device__ as
// empty before including this file.
#pragma once

#include <stdint.h>

namespace h3 {

// Attention tiling by head dim D (64, 128 or 256): a workgroup of eight
// waves owns attn_rows(D, QT) query rows of one (b, h) and walks the keys in
// kAttnSub-key sub-tiles. Each wave holds QT 16-row query tiles: four at head
// dim 64 (64 rows), two or three at 128 (32 or 48 rows, chosen per launch by
// choose_query_tiles), two at 256, where the waves work in pairs that share
// 32 rows, each wave holding half of the channels.
constexpr int kAttnSub = 32;
constexpr int attn_threads(int) { return 512; }
constexpr int attn_qt_min(int D) { return D == 64 ? 4 : 2; }
constexpr int attn_qt_max(int D) { return D == 64 ? 4 : D == 128 ? 3 : 2; }
constexpr int attn_rows(int D, int QT) { return attn_threads(D) / 64 * 16 * QT / (D == 256 ? 2 : 1); }

// Load balancing of the last, partial round of query tiles (stream-K): those
// tiles' sub-tile steps are split evenly over up to kSplitMaxBlocks
// workgroups, each taking at least kSplitMinSteps steps and touching at most
// two tiles; each writes one partial record per tile it touches and a second
// kernel merges them. A record holds the un-normalised fp32 accumulator (D/2
// values per lane) plus the lane's running max and partial row sum.
constexpr int kSplitMaxBlocks = 256;
constexpr int kSplitMinSteps = 16;
// Floats per partial record: the accumulator registers of every thread (its
// share of rows x D), then each thread's row offsets and partial sums, one
// of each per query tile. The workspace sizes every record for the largest
// query-tile count of the head dim.
constexpr int attn_part_floats(int D, int QT) {
  return (attn_rows(D, QT) * D / attn_threads(D) + 2 * QT) * attn_threads(D);
}
constexpr int attn_part_floats_max(int D) { return attn_part_floats(D, attn_qt_max(D)); }

// Partial records the forward workspace reserves for these sizes: two per
// split workgroup, for the largest split the launcher can choose (the most
// tiles: the fewest query tiles per wave).
inline int64_t split_part_slots(int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t D) {
  const int rows = attn_rows(D, attn_qt_min(D));
  const int64_t tiles = (int64_t)B * H * ((Sq + rows - 1) / rows);
  const int64_t steps = tiles * ((Sk + kAttnSub - 1) / kAttnSub);
  const int64_t blocks = steps / kSplitMinSteps < kSplitMaxBlocks ? steps / kSplitMinSteps : kSplitMaxBlocks;
  return 2 * blocks;
}

// Key-norm maxima for the a priori score bound of unnormalised inputs: one
// fp32 per chunk of kKnChunk prepared key rows of each (b, kv head).
constexpr int kKnChunk = 4096;
inline int64_t key_norm_chunks(int64_t Sk_pad) { return (Sk_pad + kKnChunk - 1) / kKnChunk; }

// Blocks are dispatched round-robin over the 8 XCDs, so block i of a range
// of n runs on XCD i%8. This bijection of [0, n) gives each XCD a contiguous
// run of work items (same head, neighbouring query blocks or steps), so its
// L2 serves one head's K/V stream.
__host__ __device__ inline int xcd_order(int i, int n) {
  const int xcd = i & 7;
  const int per = n >> 3, rem = n & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + (i >> 3);
}

// General-mode tiles in rank order (rank 0 first: under the causal mask the
// last query block, under the frame window the first or the longest), spread
// so that each XCD works on few heads and its L2 serves their shared keys.
// Workgroup bid runs on XCD bid % 8 as that XCD's (bid / 8)-th block. With
// L = lcm(nbh, 8), each head's ranks split into S = L / nbh residue classes
// mod S, and XCD x takes classes [P x, P x + P), P = L / 8 (at most two
// heads when nbh is even), its k-th block taking element k / P of class
// P x + k % P. Every XCD so sees the same mix of ranks, in increasing order.
// Ranks past the whole rows of classes (fewer than S per head) come last,
// heads inner. A bijection of [0, nq * nbh) onto (rank < nq, head < nbh).
// With per-item lengths (ragged) the heads of different items differ in
// work, so each rank keeps all of them together (heads inner) and no XCD is
// left with the short items only.
__host__ __device__ inline void spread_tile(int bid, int nq, int nbh, bool ragged, int& rank, int& bh) {
  if (ragged) {
    rank = bid / nbh;
    bh = bid - rank * nbh;
    return;
  }
  const int low = nbh & -nbh;
  const int g = low < 8 ? low : 8;
  const int64_t L = (int64_t)nbh * (8 / g);
  const int S = 8 / g, P = (int)(L / 8);
  const int R = nq / S;
  const int64_t rect = (int64_t)R * L;
  if (bid >= rect) {
    const int i = (int)(bid - rect);
    rank = R * S + i / nbh;
    bh = i - (i / nbh) * nbh;
    return;
  }
  const int x = bid & 7, k = bid >> 3;
  const int cls = x * P + k % P, e = k / P;
  bh = cls / S;
  rank = e * S + cls % S;
}

// Uniform-mode schedule of n_valid valid tiles of NU sub-tile steps each on
// `cus` compute units (one tile per CU at a time): the first n_whole tiles
// run whole; when the last round is partial, its n_split tiles' steps are
// divided over n_blocks > n_split workgroups (at most one per CU, each at
// least kSplitMinSteps steps, and at most part_slots / 2 of them, as the
// workspace holds two records per block). n_split = n_blocks = 0 when
// nothing is split.
struct SplitPlan {
  int64_t n_whole, n_split, n_blocks;
};
inline SplitPlan split_plan(int64_t n_valid, int64_t NU, int64_t cus, int64_t part_slots) {
  SplitPlan p{n_valid, 0, 0};
  if (cus > kSplitMaxBlocks) cus = kSplitMaxBlocks;
  if (cus <= 0 || NU <= 0) return p;
  const int64_t r = n_valid % cus;
  int64_t blocks = cus;
  if (r * NU / kSplitMinSteps < blocks) blocks = r * NU / kSplitMinSteps;
  if (part_slots / 2 < blocks) blocks = part_slots / 2;
  if (r > 0 && blocks > r) {
    p.n_whole = n_valid - r;
    p.n_split = r;
    p.n_blocks = blocks;
  }
  return p;
}

// Query tiles per wave for one launch (head dim 128 has two choices; the
// others one). Three tiles feed each fragment read and each direct load to a
// third more matrix-core instructions, about 5% faster per unit of work, but
// their 384-row tiles fill the rounds of the chip differently. Uniform mode
// compares the two schedules' busy time per CU (split_plan: whole rounds of
// NU steps, then the split round's steps per block, plus a fixed cost of
// kSplitOverheadSteps for its records and merge), each step weighted by its
// rows and that efficiency. General mode (tiles of unequal length, no split)
// takes three tiles when they make at least two rounds. cus <= 0 (unknown)
// takes the largest count.
constexpr int kSplitOverheadSteps = 64;
inline int choose_query_tiles(int D, bool general, int64_t BH, int64_t q_valid, int64_t NU, int64_t cus,
                              int64_t part_slots) {
  const int lo = attn_qt_min(D), hi = attn_qt_max(D);
  if (lo == hi || cus <= 0) return hi;
  const int64_t c = cus < kSplitMaxBlocks ? cus : kSplitMaxBlocks;
  if (general) {
    const int64_t rows = attn_rows(D, hi);
    return BH * ((q_valid + rows - 1) / rows) >= 2 * c ? hi : lo;
  }
  // Busy time num / den in units of (one step of a 16-row query tile) / 20:
  // a step of QT tiles costs 20 QT at three tiles and 21 QT at two. The
  // busiest CU's steps are scaled by n_blocks so the split round's share is
  // whole.
  struct Cost {
    int64_t num, den;
  };
  auto cost = [&](int QT) {
    const int64_t rows = attn_rows(D, QT);
    const int64_t n = BH * ((q_valid + rows - 1) / rows);
    const SplitPlan p = split_plan(n, NU, cus, part_slots);
    Cost r;
    if (p.n_blocks > 0) {
      r.num = (p.n_whole / c * NU + kSplitOverheadSteps) * p.n_blocks + p.n_split * NU;
      r.den = p.n_blocks;
    } else {
      r.num = (n + c - 1) / c * NU;
      r.den = 1;
    }
    r.num *= (int64_t)QT * (QT == 3 ? 20 : 21);
    return r;
  };
  const Cost a = cost(lo), b = cost(hi);
  return (__int128)b.num * a.den <= (__int128)a.num * b.den ? hi : lo;
}

// The work of split workgroup j (0 <= j < n_blocks): of the U = n_split * NU
// steps of the split tiles, steps [j U / n_blocks, (j + 1) U / n_blocks).
// Since n_blocks > n_split that range holds at most NU steps, so it touches
// split tile `tile` (its steps [xb0, xe0)) and, when nseg = 2, the first
// xe1 steps of tile + 1. The block writes record rec0 = 2j for the first
// tile and rec1 = 2j + 1 for the second.
//
// Step p of a split tile t reads key sub-tile (p - o_t) mod NU, where o_t is
// the first block start inside tile t (split_key_origin): every block that
// starts in a tile then begins at key sub-tile 0 (or, for a second start in
// the same tile, at its own length), and every block that runs into a tile
// from the previous one reads that tile's last sub-tiles. Blocks that share
// an XCD (consecutive j, one head) so stream the same keys at the same time
// and fetch them once through its L2, instead of each streaming its own
// offset. No segment wraps: the rotation's seam is a block start. The keys
// of segment 0 are [kb0, kb0 + xe0 - xb0), those of segment 1 [kb1, kb1 + xe1);
// both lie in [0, NU), and a segment holding the last sub-tile ends there.
struct SplitSeg {
  int tile, xb0, xe0, rec0, nseg, xe1, rec1, kb0, kb1;
};
__host__ __device__ inline int split_key_origin(int t, int n_split, int NU, int n_blocks) {
  const int64_t U = (int64_t)n_split * NU;
  const int64_t j = ((int64_t)t * NU * n_blocks + U - 1) / U;   // the first block with start >= t NU
  return (int)(j * U / n_blocks - (int64_t)t * NU);
}
__host__ __device__ inline SplitSeg split_segments(int j, int n_split, int NU, int n_blocks) {
  const int64_t U = (int64_t)n_split * NU;
  const int64_t s0 = (int64_t)j * U / n_blocks;
  const int64_t s1 = (int64_t)(j + 1) * U / n_blocks;
  SplitSeg sg;
  sg.tile = (int)(s0 / NU);
  sg.xb0 = (int)(s0 - (int64_t)sg.tile * NU);
  const int64_t e0 = s1 - (int64_t)sg.tile * NU;
  sg.xe0 = (int)(e0 < NU ? e0 : NU);
  sg.rec0 = 2 * j;
  sg.kb0 = sg.xb0 - split_key_origin(sg.tile, n_split, NU, n_blocks);
  sg.nseg = 1;
  sg.xe1 = 0;
  sg.rec1 = -1;
  sg.kb1 = 0;
  if (s1 > (int64_t)(sg.tile + 1) * NU) {
    sg.nseg = 2;
    sg.xe1 = (int)(s1 - (int64_t)(sg.tile + 1) * NU);
    sg.rec1 = 2 * j + 1;
    sg.kb1 = NU - split_key_origin(sg.tile + 1, n_split, NU, n_blocks);
  }
  return sg;
}

// The merge of split tile t: step x lies in block floor(((x + 1) n - 1) / U)
// (the inverse of the ranges above), so the blocks that touch tile t are
// j0 .. j1, those holding its first and last steps; block j's record for
// tile t is 2j + (t - the first tile of block j).
__host__ __device__ inline void merge_blocks(int t, int n_split, int NU, int n_blocks, int& j0, int& j1) {
  const int64_t U = (int64_t)n_split * NU;
  const int64_t x0 = (int64_t)t * NU, x1 = x0 + NU - 1;
  j0 = (int)(((x0 + 1) * n_blocks - 1) / U);
  j1 = (int)(((x1 + 1) * n_blocks - 1) / U);
}
__host__ __device__ inline int merge_record(int j, int t, int n_split, int NU, int n_blocks) {
  const int64_t U = (int64_t)n_split * NU;
  const int first = (int)(((int64_t)j * U / n_blocks) / NU);
  return 2 * j + (t - first);
}

// Frame window, longest-first order: the most query blocks per head that are
// ranked, and the ranking key of query block j with xe sub-tiles: the
// sub-tile count above, kWinOrderMax - 1 - j below, plus one (so a padding
// key of zero is below them all). Keys are unique, so the block of rank r
// is the one with exactly r larger keys, and ranks are a permutation.
constexpr int kWinOrderMax = 1024;
__host__ __device__ inline uint32_t win_rank_key(int xe, int j) {
  const int x = xe < (1 << 21) - 1 ? xe : (1 << 21) - 1;
  return ((uint32_t)x << 10 | (uint32_t)(kWinOrderMax - 1 - j)) + 1u;
}

// Frame window (row or key i in frame i / F; frames below A are anchor
// frames whose rows see every key; frame f >= A is in chunk (f - A) / C and
// its rows see the anchor frames and the chunks within R of their own): the
// sub-tiles of the query tile at rows [q00, q00 + BM) with qv valid rows and
// kvv valid keys. They are [0, wn1) (the anchor frames, or every key when
// the tile has a dense row) then [wn1 + ws2, xe + ws2) (the union of its
// rows' chunk windows), merged when they touch, so virtual step v < xe reads
// sub-tile v (v < wn1) or v + ws2. fast: every row of the tile sees the same
// whole sub-tiles (only a partial last sub-tile at kvv needs a mask). cap:
// the chunks that can hold keys, plus one. Requires q00 < qv and kvv >= 1.
struct WinSpan {
  int wn1, ws2, xe, cap;
  bool fast;
};
__host__ __device__ inline WinSpan win_span(int F, int C, int R, int A, int BM, int q00, int qv, int kvv) {
  auto imin = [](int x, int y) { return x < y ? x : y; };
  auto imax = [](int x, int y) { return x > y ? x : y; };
  WinSpan w;
  w.cap = (kvv + F - 1) / F / C + 1;
  w.fast = true;
  const int q1 = imin(q00 + BM, qv);
  const int f0 = q00 / F, f1 = (q1 - 1) / F;
  int hi1, lo2 = 0, hi2 = 0;
  if (f0 < A) {
    hi1 = kvv;
    w.fast = f1 < A;
  } else {
    const int c0 = (f0 - A) / C, c1 = (f1 - A) / C;
    hi1 = imin(A * F, kvv);
    lo2 = imin((A + C * imax(c0 - R, 0)) * F, kvv);
    hi2 = imin((A + C * imin(c1 + R + 1, w.cap)) * F, kvv);
    w.fast = c0 == c1 && (hi1 % kAttnSub == 0 || hi1 == kvv) && lo2 % kAttnSub == 0 &&
             (hi2 % kAttnSub == 0 || hi2 == kvv);
  }
  int s1 = (hi1 + kAttnSub - 1) / kAttnSub;
  int s2lo = lo2 / kAttnSub, s2hi = (hi2 + kAttnSub - 1) / kAttnSub;
  if (hi2 <= lo2) s2lo = s2hi = s1;   // no window key below kvv
  if (s2lo <= s1) {                   // the ranges touch or overlap: one range
    s1 = imax(s1, s2hi);
    s2lo = s2hi = s1;
  }
  w.wn1 = s1;
  w.ws2 = s2lo - s1;   // sub-tile of virtual step v >= wn1 is v + ws2
  w.xe = s1 + (s2hi - s2lo);
  return w;
}

}  // namespace h3
