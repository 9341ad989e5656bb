// Key-range and tile-class helpers shared by the host (tests, launch sizing)
// and the device (per-tile loop bounds and mask decisions).
//
// A query at token index t of a sequence with Lq queries and Lk keys sits at
// key-axis position p = t + (Lk - Lq) (bottom-right alignment: the queries are
// the last Lq tokens of the sequence; "FA4 (CuTeDSL) and engineering
// interfaces", section 6.2, and "Attention kernels: FlashAttention and
// PagedAttention", section 5.1).  It sees key j iff
//     0 <= j < Lk
//     and (not causal or j <= p)
//     and (window_left  < 0 or j >= p - window_left)
//     and (window_right < 0 or j <= p + window_right)
// (window bounds inclusive, "FA4 ...", section 7 table).
//
// Whole key tiles outside every row's range are skipped, tiles inside every
// row's range run without an element mask, and only tiles cut by a boundary
// are masked element by element ("Attention kernels ...", sections 7.2 and
// 7.3: causal halves the work, a window makes it O(N * W)).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD static inline
#endif

// Tile class bits.
enum {
  FA_TILE_VISIBLE = 1,     // some valid row sees some key of the tile
  FA_TILE_MASK_RIGHT = 2,  // cut by the causal diagonal, the right window edge or Lk
  FA_TILE_MASK_LEFT = 4,   // cut by the left window edge
};

struct FaRowSpan {
  int64_t pos_lo, pos_hi;  // key-axis positions of the tile's first and last valid row
};

FA_HD int64_t fa_min64(int64_t a, int64_t b) { return a < b ? a : b; }
FA_HD int64_t fa_max64(int64_t a, int64_t b) { return a > b ? a : b; }

// Effective right bound relative to the query position: causal clamps it to 0
// (a non-negative right window is then implied by causality).
// Returns 1 and sets *right if the right side is bounded, else returns 0.
FA_HD int fa_right_bound(int causal, int wr, int64_t* right) {
  if (causal) {
    *right = 0;
    return 1;
  }
  if (wr >= 0) {
    *right = wr;
    return 1;
  }
  *right = 0;
  return 0;
}

// Inclusive key range [k_lo, k_hi] seen by at least one row of the span.
// Returns 0 when no row sees any key.
FA_HD int fa_key_range(FaRowSpan s, int64_t Lk, int causal, int wl, int wr, int64_t* k_lo,
                       int64_t* k_hi) {
  int64_t lo = 0, hi = Lk - 1, right;
  if (wl >= 0) lo = fa_max64(lo, s.pos_lo - wl);
  if (fa_right_bound(causal, wr, &right)) hi = fa_min64(hi, s.pos_hi + right);
  *k_lo = lo;
  *k_hi = hi;
  return hi >= lo;
}

// Key tiles [*n_lo, *n_hi) of width bn that the span has to visit.
FA_HD void fa_key_tiles(FaRowSpan s, int64_t Lk, int causal, int wl, int wr, int bn, int* n_lo,
                        int* n_hi) {
  int64_t lo, hi;
  if (!fa_key_range(s, Lk, causal, wl, wr, &lo, &hi)) {
    *n_lo = 0;
    *n_hi = 0;
    return;
  }
  *n_lo = (int)(lo / bn);
  *n_hi = (int)(hi / bn) + 1;
}

// Key tiles [*f_lo, *f_hi) that every row of the span sees in full (class
// FA_TILE_VISIBLE with no mask bit); empty as [0, 0).  A tile is full when its
// first key is at or right of the span's tightest left bound and its last key
// at or left of the tightest right bound.
FA_HD void fa_full_tiles(FaRowSpan s, int64_t Lk, int causal, int wl, int wr, int bn, int* f_lo,
                         int* f_hi) {
  int64_t left = 0, right_key = Lk - 1, right;
  if (wl >= 0) left = fa_max64(left, s.pos_hi - wl);
  if (fa_right_bound(causal, wr, &right)) right_key = fa_min64(right_key, s.pos_lo + right);
  const int64_t lo = (left + bn - 1) / bn;
  const int64_t hi = right_key + 1 > 0 ? (right_key + 1) / bn : 0;
  if (hi <= lo) {
    *f_lo = 0;
    *f_hi = 0;
    return;
  }
  *f_lo = (int)lo;
  *f_hi = (int)hi;
}

// Class bits of key tile n (keys [n*bn, n*bn + bn)) for the span.
FA_HD int fa_tile_class(FaRowSpan s, int64_t Lk, int causal, int wl, int wr, int bn, int n) {
  int64_t t0 = (int64_t)n * bn, t1 = t0 + bn - 1, lo, hi, right;
  int cls = 0;
  if (!fa_key_range(s, Lk, causal, wl, wr, &lo, &hi)) return 0;
  if (t1 < lo || t0 > hi) return 0;
  cls = FA_TILE_VISIBLE;
  // right side: every row must see the tile's last key
  if (t1 > Lk - 1) cls |= FA_TILE_MASK_RIGHT;
  if (fa_right_bound(causal, wr, &right) && t1 > s.pos_lo + right) cls |= FA_TILE_MASK_RIGHT;
  // left side: every row must see the tile's first key
  if (wl >= 0 && t0 < s.pos_hi - wl) cls |= FA_TILE_MASK_LEFT;
  return cls;
}

// Queries that see at least one key of [j_lo, j_hi] (inclusive, inside [0, Lk)):
// the query rows [*i_lo, *i_hi) of Lq (empty when *i_lo >= *i_hi).  The
// backward's key-block tiles loop over these (the transpose of the key range
// of a row span).  Query t sits at p = t + Lk - Lq; it needs some key j of the
// block with j <= p (causal) or j <= p + wr (right window) and j >= p - wl
// (left window).
FA_HD void fa_query_range(int64_t j_lo, int64_t j_hi, int64_t Lq, int64_t Lk, int causal, int wl, int wr,
                          int64_t* i_lo, int64_t* i_hi) {
  const int64_t off = Lk - Lq;
  int64_t lo = 0, hi = Lq;
  if (causal)
    lo = j_lo - off;  // p >= j_lo (binds before any right window, which only adds p + wr >= j)
  else if (wr >= 0)
    lo = j_lo - wr - off;  // p + wr >= j_lo
  if (wl >= 0) hi = j_hi + wl - off + 1;  // p - wl <= j_hi
  *i_lo = fa_max64(lo, 0);
  *i_hi = fa_min64(hi, Lq);
}
