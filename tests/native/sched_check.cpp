// Host build of the kernels' scheduler header: checks the int32 closed-form
// full-tile test against the int64 tile ranges over an exhaustive grid of
// small shapes, the per-block skip tests against cell enumeration, and the
// launch-id decode's multiply-high division against plain division. Exit
// status 0 = all agree.
#include <cstdio>
#include <initializer_list>
#include <vector>

#include "../../sliding_window_flash_amd/csrc/sched.hpp"

int main() {
  long checked = 0, bad = 0;
  const int wins[] = {1, 2, 3, 5, 31, 32, 33, 64, 127, 128, 129, 1000, 2147483647};
  for (int lq = 0; lq <= 140; lq += 7)
    for (int dl = -70; dl <= 70; dl += 35)
      for (int w : wins)
        for (int causal = 0; causal <= 1; ++causal) {
          const int lk = lq + dl;
          if (lk < 0) continue;
          const swa::SeqGeom g{lq, lk, w, causal != 0};
          for (int bm : {16, 32, 64})
            for (int bn : {16, 32, 64, 128})
              for (int qb = 0; qb * bm < lq; ++qb)
                for (int kb = 0; kb * bn < lk; ++kb) {
                  const bool a = swa::tile_is_full(g, qb, bm, kb, bn);
                  const bool b = swa::tile_full_i32(lq, lk, w, causal != 0, qb, bm, kb, bn);
                  ++checked;
                  if (a != b) {
                    if (bad < 5)
                      printf("mismatch lq=%d lk=%d w=%d causal=%d bm=%d bn=%d qb=%d kb=%d: %d vs %d\n", lq,
                             lk, w, causal, bm, bn, qb, kb, a, b);
                    ++bad;
                  }
                }
        }
  // block_masked against cell-by-cell enumeration (the kernels' per-wave skip)
  long bchecked = 0, bbad = 0;
  for (int lq = 1; lq <= 140; lq += 9)
    for (int dl = -70; dl <= 70; dl += 35)
      for (int w : wins)
        for (int causal = 0; causal <= 1; ++causal) {
          const int lk = lq + dl;
          if (lk < 0) continue;
          const swa::SeqGeom g{lq, lk, w, causal != 0};
          for (int rows : {32})
            for (int cols : {32, 64})
              for (int a = 0; a < lq + rows; a += 16)
                for (int b = 0; b < lk + cols; b += 16) {
                  bool any = false;
                  for (int i = a; i < a + rows && !any; ++i)
                    for (int j = b; j < b + cols && !any; ++j) any = swa::cell_visible(g, i, j);
                  const bool m = swa::block_masked(lq, lk, w, causal != 0, a, rows, b, cols);
                  ++bchecked;
                  if (m == any) {
                    if (bbad < 5)
                      printf("block mismatch lq=%d lk=%d w=%d causal=%d a=%d b=%d rows=%d cols=%d: masked=%d visible=%d\n",
                             lq, lk, w, causal, a, b, rows, cols, m, any);
                    ++bbad;
                  }
                }
        }
  printf("blocks checked %ld, mismatches %ld\n", bchecked, bbad);
  bad += bbad;
  // the per-key-block intervals of query tiles against the per-step tests
  // they replace: block_seen_query_tiles == !block_masked and
  // key_tile_full_query_tiles == tile_full_i32, for every query tile
  long ichecked = 0, ibad = 0;
  for (int lq = 0; lq <= 200; lq += 7)
    for (int dl : {-130, -37, -1, 0, 1, 37, 130})
      for (int w : wins)
        for (int causal = 0; causal <= 1; ++causal) {
          const int lk = lq + dl;
          if (lk < 0) continue;
          const swa::SeqGeom g{lq, lk, w, causal != 0};
          for (int bm : {32, 64})
            for (int bn : {32, 64, 128})
              for (int kb = 0; kb * bn < lk; ++kb) {
                const swa::QbRange f = swa::key_tile_full_query_tiles(g, kb, bn, bm);
                for (int qb = 0; qb * bm < lq + bm; ++qb) {
                  const bool want = qb * bm < lq && swa::tile_full_i32(lq, lk, w, causal != 0, qb, bm, kb, bn);
                  const bool got = f.lo <= qb && qb <= f.hi;
                  ++ichecked;
                  if (want != got) {
                    if (ibad < 5)
                      printf("full-range mismatch lq=%d lk=%d w=%d causal=%d bm=%d bn=%d kb=%d qb=%d: %d vs %d [%d,%d]\n",
                             lq, lk, w, causal, bm, bn, kb, qb, want, got, f.lo, f.hi);
                    ++ibad;
                  }
                }
                for (int r0 : {0, 32})
                  for (int c : {0, 32, 96})
                    for (int rows : {32})
                      for (int cols : {32}) {
                        if (r0 + rows > bm || c + cols > bn) continue;
                        const int c0 = kb * bn + c;
                        const swa::QbRange v = swa::block_seen_query_tiles(g, bm, r0, rows, c0, cols);
                        for (int qb = 0; qb * bm < lq + bm; ++qb) {
                          const bool want = !swa::block_masked(lq, lk, w, causal != 0, qb * bm + r0, rows, c0, cols);
                          const bool got = v.lo <= qb && qb <= v.hi;
                          ++ichecked;
                          if (want != got) {
                            if (ibad < 5)
                              printf("seen-range mismatch lq=%d lk=%d w=%d causal=%d bm=%d r0=%d c0=%d qb=%d: %d vs %d [%d,%d]\n",
                                     lq, lk, w, causal, bm, r0, c0, qb, want, got, v.lo, v.hi);
                            ++ibad;
                          }
                        }
                      }
              }
        }
  printf("intervals checked %ld, mismatches %ld\n", ichecked, ibad);
  bad += ibad;
  // the launch-id decode's division by multiply-high against plain division:
  // every numerator below 2^17 for every divisor up to 4,100; for divisors
  // up to 2^31 - 1 (small, powers of two and their neighbours, large primes,
  // pseudo-random), the multiples of d and their neighbours across [0, 2^31)
  // and pseudo-random numerators
  long fchecked = 0, fbad = 0;
  auto check_div = [&](uint32_t d, uint32_t n) {
    const swa::FastDiv f = swa::make_fast_div(d);
    const uint32_t got = swa::fast_div(n, f), want = n / d;
    ++fchecked;
    if (got != want) {
      if (fbad < 5) printf("fast_div mismatch n=%u d=%u: %u vs %u\n", n, d, got, want);
      ++fbad;
    }
  };
  for (uint32_t d = 1; d <= 4100; ++d)
    for (uint32_t n = 0; n < (1u << 17); ++n) check_div(d, n);
  uint64_t x = 0x9E3779B97F4A7C15ull;
  auto rnd = [&]() {
    x ^= x << 13;
    x ^= x >> 7;
    x ^= x << 17;
    return x;
  };
  std::vector<uint32_t> divisors;
  for (int k = 0; k < 31; ++k)
    for (int e = -1; e <= 1; ++e) {
      const int64_t d = ((int64_t)1 << k) + e;
      if (d >= 1 && d < ((int64_t)1 << 31)) divisors.push_back((uint32_t)d);
    }
  for (uint32_t d : {3u, 7u, 10u, 641u, 6700417u, 65537u, 2147483647u, 2147483629u, 1000003u, 12345u}) divisors.push_back(d);
  for (int i = 0; i < 200; ++i) divisors.push_back((uint32_t)(1 + rnd() % 2147483647ull));
  for (uint32_t d : divisors) {
    const uint32_t top = 2147483647u;
    for (uint64_t k = 0; k * d <= top; k += (top / d) / 64 + 1)
      for (int e = -1; e <= 1; ++e) {
        const int64_t n = (int64_t)(k * d) + e;
        if (n >= 0 && n <= top) check_div(d, (uint32_t)n);
      }
    check_div(d, top);
    for (int i = 0; i < 2000; ++i) check_div(d, (uint32_t)(rnd() & 0x7fffffffu));
  }
  printf("divisions checked %ld, mismatches %ld\n", fchecked, fbad);
  bad += fbad;
  printf("checked %ld, mismatches %ld\n", checked, bad);
  return bad != 0;
}
