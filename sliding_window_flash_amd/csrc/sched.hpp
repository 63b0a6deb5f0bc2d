// Block-range scheduler: which tiles of the score matrix a kernel visits.
//
// "Off NVIDIA, you fix the platform yourself", section "What did fixing it
// take?": the tiled backward must skip blocks lying entirely outside the
// window and mask only the cells on its edge; the first block a query visits
// is no longer block zero, and some key blocks are never visited.
//
// Integer code only, compiled for both the host (CPU tests and the C ABI's
// inspection calls) and the device (every kernel). All position arithmetic is
// int64 so that window = INT32_MAX and 32-bit lengths cannot overflow.
//
// Geometry of one sequence: L_q queries, L_k keys, delta = L_k - L_q >= 0;
// query i sits at key position p = i + delta. Causal cell (i, j) is visible
// iff j <= p and p - j < window. Without the causal mask the window is
// two-sided: visible iff |p - j| < window (window >= L_k: every cell).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SWA_HD __host__ __device__ inline
#else
#define SWA_HD inline
#endif

namespace swa {

struct SeqGeom {
  int64_t lq, lk, window;
  bool causal;
  SWA_HD int64_t delta() const { return lk - lq; }
};

struct TileRange {
  int32_t lo, hi;            // visited tiles [lo, hi]; empty when lo > hi
  int32_t full_lo, full_hi;  // tiles with every cell visible; empty when full_lo > full_hi
};

SWA_HD int64_t floor_div(int64_t a, int64_t b) {  // b > 0
  return a >= 0 ? a / b : -((-a + b - 1) / b);
}

// Query tile qb (rows [qb*bm, min(lq, qb*bm+bm)) ) -> key tiles of size bn.
SWA_HD TileRange query_tile_keys(const SeqGeom& s, int32_t qb, int32_t bm, int32_t bn) {
  TileRange r{0, -1, 0, -1};
  const int64_t i0 = (int64_t)qb * bm;
  int64_t i1 = i0 + bm - 1;
  if (i1 > s.lq - 1) i1 = s.lq - 1;
  if (i0 > i1 || s.lk <= 0) return r;
  int64_t jlo, jhi;
  if (s.causal) {
    const int64_t pmin = i0 + s.delta(), pmax = i1 + s.delta();
    jlo = pmin - s.window + 1;
    if (jlo < 0) jlo = 0;
    jhi = pmax < s.lk - 1 ? pmax : s.lk - 1;
    if (jlo > jhi) return r;
    r.lo = (int32_t)(jlo / bn);
    r.hi = (int32_t)(jhi / bn);
    // full tile kb: kb*bn+bn-1 <= pmin (causal), pmax - kb*bn < window (window),
    // kb*bn+bn <= lk (in bounds), and the query tile has all bm rows.
    if (i1 - i0 + 1 == bm) {
      const int64_t fhi_causal = floor_div(pmin + 1, bn) - 1;
      const int64_t fhi_bound = s.lk / bn - 1;
      int64_t fhi = fhi_causal < fhi_bound ? fhi_causal : fhi_bound;
      // pmax - kb*bn < window  <=>  kb*bn > pmax - window  <=>  kb >= floor((pmax-window)/bn)+1
      int64_t flo = floor_div(pmax - s.window, bn) + 1;
      if (flo < r.lo) flo = r.lo;
      if (fhi > r.hi) fhi = r.hi;
      if (flo <= fhi) {
        r.full_lo = (int32_t)flo;
        r.full_hi = (int32_t)fhi;
      }
    }
  } else {
    // two-sided: keys within window - 1 of some row's position
    const int64_t pmin = i0 + s.delta(), pmax = i1 + s.delta();
    jlo = pmin - s.window + 1;
    if (jlo < 0) jlo = 0;
    jhi = pmax + s.window - 1;
    if (jhi > s.lk - 1) jhi = s.lk - 1;
    if (jlo > jhi) return r;
    r.lo = (int32_t)(jlo / bn);
    r.hi = (int32_t)(jhi / bn);
    // full tile kb: kb*bn >= pmax - window + 1, kb*bn + bn - 1 <= pmin + window - 1,
    // kb*bn + bn <= lk, and the query tile has all bm rows
    if (i1 - i0 + 1 == bm) {
      int64_t flo = -floor_div(-(pmax - s.window + 1), bn);  // ceil
      int64_t fhi = floor_div(pmin + s.window - bn, bn);
      const int64_t fhi_bound = s.lk / bn - 1;
      if (fhi > fhi_bound) fhi = fhi_bound;
      if (flo < r.lo) flo = r.lo;
      if (fhi > r.hi) fhi = r.hi;
      if (flo <= fhi) {
        r.full_lo = (int32_t)flo;
        r.full_hi = (int32_t)fhi;
      }
    }
  }
  return r;
}

// Key tile kb (cols [kb*bn, min(lk, kb*bn+bn)) ) -> query tiles of size bm that
// see at least one of its cells. Empty (lo > hi) when no query sees it.
SWA_HD TileRange key_tile_queries(const SeqGeom& s, int32_t kb, int32_t bn, int32_t bm) {
  TileRange r{0, -1, 0, -1};
  const int64_t j0 = (int64_t)kb * bn;
  int64_t j1 = j0 + bn - 1;
  if (j1 > s.lk - 1) j1 = s.lk - 1;
  if (j0 > j1 || s.lq <= 0) return r;
  int64_t ilo, ihi;
  if (s.causal) {
    // visible iff i >= j - delta and i <= j - delta + window - 1
    ilo = j0 - s.delta();
    if (ilo < 0) ilo = 0;
    ihi = j1 - s.delta() + s.window - 1;
    if (ihi > s.lq - 1) ihi = s.lq - 1;
  } else {
    // two-sided: p within window - 1 of some key of the tile
    ilo = j0 - s.window + 1 - s.delta();
    if (ilo < 0) ilo = 0;
    ihi = j1 + s.window - 1 - s.delta();
    if (ihi > s.lq - 1) ihi = s.lq - 1;
  }
  if (ilo > ihi) return r;
  r.lo = (int32_t)(ilo / bm);
  r.hi = (int32_t)(ihi / bm);
  return r;
}

// Workgroups are handed to the 8 XCDs round-robin (id % 8), each XCD with its
// own L2. Map launch id -> logical work id so that XCD x runs the contiguous
// logical range [x*n/8, (x+1)*n/8) (remainder spread over the first XCDs):
// neighbouring logical items, which share K/V rows, then share an L2. Any
// bijection is correct; this one only decides locality.
SWA_HD int32_t xcd_remap(int32_t id, int32_t n, int32_t nxcd = 8) {
  const int32_t xcd = id % nxcd, slot = id / nxcd;
  const int32_t per = n / nxcd, rem = n % nxcd;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Division by a divisor d >= 1 that is fixed for a launch, as a multiply-high,
// an add and a shift (Granlund and Montgomery, "Division by invariant integers
// using multiplication", 1994, section 4): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, which is below 2^32, floor(n / d) is
// (mulhi(m, n) + n) >> l for every 32-bit n. For n < 2^31, as in the kernels'
// launch-id decode, the sum cannot overflow (mulhi(m, n) <= n). The launchers
// build the multipliers once per launch on the host; a workgroup then decodes
// its launch id without the long sequence of a runtime 32-bit division.
struct FastDiv {
  uint32_t d, m, l;
};
SWA_HD FastDiv make_fast_div(uint32_t d) {  // 1 <= d < 2^31, so that l <= 31
  uint32_t l = 0;
  while (((uint64_t)1 << l) < d) ++l;
  const uint64_t m = ((uint64_t)1 << 32) * (((uint64_t)1 << l) - d) / d + 1;
  return FastDiv{d, (uint32_t)m, l};
}
SWA_HD uint32_t fast_div(uint32_t n, const FastDiv& f) {  // floor(n / f.d) for n < 2^31
  const uint32_t hi = (uint32_t)(((uint64_t)f.m * n) >> 32);
  return (hi + n) >> f.l;
}

// Per-cell visibility by the definition. The kernels mask edge tiles with bit
// runs built from the same rule; the host checks enumerate cells with this.
SWA_HD bool cell_visible(const SeqGeom& s, int64_t i, int64_t j) {
  if (i >= s.lq || j >= s.lk) return false;
  const int64_t p = i + s.delta();
  if (!s.causal) return p - j < s.window && j - p < s.window;
  return j <= p && p - j < s.window;
}

// The same test in int32 closed form, for the kernels' inner loops: every
// cell of (query tile qb, key tile kb) is visible iff the query tile has all bm
// rows, the key tile all bn keys, and (causal) its last key is <= the first
// query's position and the last query's position minus its first key is
// < window. Requires positions < 2^31 (guaranteed by the ABI's int32 sizes).
SWA_HD bool tile_full_i32(int32_t lq, int32_t lk, int32_t window, bool causal, int32_t qb,
                          int32_t bm, int32_t kb, int32_t bn) {
  const int32_t i0 = qb * bm, j0 = kb * bn, delta = lk - lq;
  if (i0 + bm > lq || j0 + bn > lk) return false;
  // differences of positions lie in (-2^31, 2^31): no overflow
  if (!causal) return (i0 + bm - 1 + delta) - j0 < window && (j0 + bn - 1) - (i0 + delta) < window;
  return j0 + bn - 1 <= i0 + delta && (i0 + bm - 1 + delta) - j0 < window;
}

// Is every cell of the block (queries [a, a + rows), keys [b, b + cols)) of one
// sequence masked? Then the block contributes nothing (P = 0, dS = 0) and a
// wave may skip it. Causal: the block's first key lies after its last query's
// position, or its last key lies at or beyond the window of its first query.
// Rows past L_q and keys past L_k are masked. int64 arithmetic: window may be
// INT32_MAX.
SWA_HD bool block_masked(int32_t lq, int32_t lk, int32_t window, bool causal, int32_t a, int32_t rows,
                         int32_t b, int32_t cols) {
  if (a >= lq || b >= lk) return true;
  const int64_t delta = (int64_t)lk - lq;
  const int64_t p_last = (int64_t)(a + rows - 1 < lq - 1 ? a + rows - 1 : lq - 1) + delta;
  const int64_t p_first = (int64_t)a + delta;
  const int64_t b_last = (int64_t)(b + cols - 1 < lk - 1 ? b + cols - 1 : lk - 1);
  const bool too_old = p_first - b_last >= (int64_t)window;  // every key older than every row's window
  if (!causal) return too_old || (int64_t)b - p_last >= (int64_t)window;
  return (int64_t)b > p_last || too_old;
}

SWA_HD int64_t ceil_div(int64_t a, int64_t b) { return -floor_div(-a, b); }  // b > 0

struct QbRange {
  int32_t lo, hi;  // query tiles [lo, hi]; empty when lo > hi
};

// Query tiles qb (of bm rows) for which the block of rows [qb*bm + r0,
// qb*bm + r0 + rows) and keys [c0, c0 + cols) of one sequence holds at least
// one visible cell: exactly the qb for which block_masked() is false. Keys
// [c0, b_last] are visible to rows [c0 - delta, b_last - delta + window - 1]
// (causal) or [c0 - delta - window + 1, b_last - delta + window - 1]
// (two-sided), clipped to [0, L_q); the block's rows meet that interval for a
// contiguous run of qb. Computed once per key block, it replaces a per-step
// test by two compares.
SWA_HD QbRange block_seen_query_tiles(const SeqGeom& s, int32_t bm, int32_t r0, int32_t rows, int32_t c0,
                                      int32_t cols) {
  QbRange r{0, -1};
  if (c0 >= s.lk || s.lq <= 0 || rows <= 0 || cols <= 0) return r;
  const int64_t b_last = (int64_t)c0 + cols - 1 < s.lk - 1 ? (int64_t)c0 + cols - 1 : s.lk - 1;
  int64_t ilo = s.causal ? (int64_t)c0 - s.delta() : (int64_t)c0 - s.delta() - s.window + 1;
  int64_t ihi = b_last - s.delta() + s.window - 1;
  if (ilo < 0) ilo = 0;
  if (ihi > s.lq - 1) ihi = s.lq - 1;
  if (ilo > ihi) return r;
  int64_t lo = ceil_div(ilo - r0 - rows + 1, bm), hi = floor_div(ihi - r0, bm);
  if (lo < 0) lo = 0;
  if (lo > hi) return r;
  r.lo = (int32_t)lo;
  r.hi = (int32_t)hi;
  return r;
}

// Query tiles qb (of bm rows) for which tile (qb, key tile kb of bn keys) has
// every cell visible: exactly the qb for which tile_full_i32() is true. All bm
// rows and bn keys must exist; causal: kb*bn + bn - 1 <= qb*bm + delta and
// qb*bm + bm - 1 + delta - kb*bn < window; two-sided: the second condition and
// kb*bn + bn - 1 - (qb*bm + delta) < window.
SWA_HD QbRange key_tile_full_query_tiles(const SeqGeom& s, int32_t kb, int32_t bn, int32_t bm) {
  QbRange r{0, -1};
  const int64_t j0 = (int64_t)kb * bn;
  if (j0 + bn > s.lk || s.lq < bm) return r;
  int64_t lo = s.causal ? ceil_div(j0 + bn - 1 - s.delta(), bm) : ceil_div(j0 + bn - s.delta() - s.window, bm);
  int64_t hi = floor_div(j0 + s.window - bm - s.delta(), bm);
  const int64_t hi_rows = floor_div(s.lq - bm, bm);
  if (hi > hi_rows) hi = hi_rows;
  if (lo < 0) lo = 0;
  if (lo > hi) return r;
  r.lo = (int32_t)lo;
  r.hi = (int32_t)hi;
  return r;
}

// Is tile (query tile qb, key tile kb) free of masked cells?
SWA_HD bool tile_is_full(const SeqGeom& s, int32_t qb, int32_t bm, int32_t kb, int32_t bn) {
  const TileRange r = query_tile_keys(s, qb, bm, bn);
  return r.full_lo <= kb && kb <= r.full_hi;
}

}  // namespace swa
