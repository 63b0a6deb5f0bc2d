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
  printf("checked %ld, mismatches %ld\n", checked, bad);
  return bad != 0;
}
