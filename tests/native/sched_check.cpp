// Host build of the kernels' scheduler header: checks the int32 closed-form
// full-tile test against the int64 tile ranges over an exhaustive grid of
// small shapes. Exit status 0 = all agree.
#include <cstdio>
#include <initializer_list>

#include "../../sliding_window_flash_amd/csrc/sched.hpp"

int main() {
  long checked = 0, bad = 0;
  const int wins[] = {1, 2, 3, 5, 31, 32, 33, 64, 127, 128, 129, 1000, 2147483647};
  for (int lq = 0; lq <= 140; lq += 7)
    for (int dl = 0; dl <= 70; dl += 35)
      for (int w : wins)
        for (int causal = 0; causal <= 1; ++causal) {
          const int lk = lq + dl;
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
    for (int dl = 0; dl <= 70; dl += 35)
      for (int w : wins)
        for (int causal = 0; causal <= 1; ++causal) {
          const int lk = lq + dl;
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
    for (int dl : {0, 1, 37, 130})
      for (int w : wins)
        for (int causal = 0; causal <= 1; ++causal) {
          const int lk = lq + dl;
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
  printf("checked %ld, mismatches %ld\n", checked, bad);
  return bad != 0;
}
