"""The edge-tile masks of the attention kernels, compiled for the host.

Inside an edge tile the kernels build each lane's visibility as one run of bits
(row_window / pair_window and the bit-run helpers in attn_kernels.hip) and
mask cell o of the lane's block by bit o. This test compiles exactly that part
of the kernel source with g++, expands the bits into the cells the kernels'
register layout assigns them (offset 32 kt + 8 (r / 4) + r % 4 from the lane's
base, lanes of both halves), and compares every cell with the oracle's
visibility matrix: causal, two-sided and full windows, L_q < L_k and L_q > L_k,
ragged tails. Padding cells (keys past L_k in a query-major tile, rows past L_q in a
key-major block) must come out masked, since their operands arrive as zeros."""
import ctypes
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle.dense import visible_cells
from sliding_window_flash_amd.workloads import INT32_MAX

SRC = os.path.join(os.path.dirname(__file__), "..", "sliding_window_flash_amd", "csrc", "attn_kernels.hip")
BEGIN = "// Per-query visibility as one unsigned range test"
END = "// s[r] (offset o = 8 (r / 4) + r % 4 in the lane's 32-cell block)"

HOST = r'''
#include <cstdint>
#include <algorithm>
using std::min; using std::max;
#define __device__
#define __forceinline__ inline
static inline uint32_t min(uint32_t a, uint32_t b) { return a < b ? a : b; }
%s
static inline int cell_off(int kt, int r) { return 32 * kt + 8 * (r >> 2) + (r & 3); }
extern "C" {
// query-major (forward, dQ): 64-key tiles; out[i * (nkb * 64) + key], rows i < lq
void qm_cells(int lq, int lk, int window, int causal, uint8_t* out) {
  const int nkb = (lk + 63) / 64, ld = nkb * 64;
  for (int i = 0; i < lq; ++i) {
    const RowWindow rw = row_window(i + lk - lq, lq, lk, window, causal != 0);
    for (int kb = 0; kb < nkb; ++kb)
      for (int half = 0; half < 2; ++half) {
        const int jb = kb * 64 + 4 * half;
        const uint64_t vis = row_keys_visible(rw.mpos - (uint32_t)jb, rw.mlim, rw.pad_keys ? max(lk - jb, 0) : -1);
        for (int kt = 0; kt < 2; ++kt)
          for (int r = 0; r < 16; ++r) {
            const int o = cell_off(kt, r);
            out[(int64_t)i * ld + jb + o] = (uint8_t)((vis >> o) & 1u);
          }
      }
  }
}
// key-major (dK/dV): 32-row query blocks; out[i * lk + j], keys j < lk, rows i < nqb * 32
void km_cells(int lq, int lk, int window, int causal, uint8_t* out) {
  const PairWindow pw = pair_window(lq, lk, window, causal != 0);
  const int nqb = (lq + 31) / 32;
  for (int j = 0; j < lk; ++j)
    for (int qb = 0; qb < nqb; ++qb)
      for (int half = 0; half < 2; ++half) {
        const int ib = qb * 32 + 4 * half;
        const uint32_t vis = key_rows_visible(ib, ib + (lk - lq) - j + pw.off, lq, pw);
        for (int r = 0; r < 16; ++r) {
          const int o = cell_off(0, r);
          out[(int64_t)(ib + o) * lk + j] = (uint8_t)((vis >> o) & 1u);
        }
      }
}
}
'''


@pytest.fixture(scope="module")
def masks_lib():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    text = open(SRC).read()
    a, b = text.index(BEGIN), text.index(END)
    d = tempfile.mkdtemp(prefix="edge_masks_")
    src, so = os.path.join(d, "m.cpp"), os.path.join(d, "m.so")
    with open(src, "w") as f:
        f.write(HOST % text[a:b])
    subprocess.run([gxx, "-O2", "-std=c++17", "-shared", "-fPIC", "-o", so, src], check=True)
    lib = ctypes.CDLL(so)
    for fn in (lib.qm_cells, lib.km_cells):
        fn.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p]
        fn.restype = None
    yield lib
    shutil.rmtree(d, ignore_errors=True)


CASES = [
    # lq, lk, window, causal
    (200, 200, 1, True), (200, 200, 31, True), (200, 200, 32, True), (200, 200, 33, True),
    (200, 200, 64, True), (200, 200, 65, True), (300, 300, 100, True), (130, 130, INT32_MAX, True),
    (70, 333, 40, True), (5, 300, 3, True), (1, 97, 97, True), (257, 257, 128, True),
    (200, 200, 1, False), (200, 200, 33, False), (200, 200, 100, False), (70, 333, 40, False),
    (130, 190, INT32_MAX, False), (190, 190, 189, False), (190, 190, 190, False), (64, 300, 65, False),
    # more queries than keys: the first L_q - L_k rows sit at negative positions
    (400, 100, 64, True), (300, 50, INT32_MAX, True), (130, 1, 1, True), (257, 200, 33, True),
    (300, 50, 64, False), (300, 50, 250, False), (97, 5, 3, False), (200, 130, INT32_MAX, False),
]


@pytest.mark.parametrize("lq,lk,window,causal", CASES)
def test_edge_masks_match_visibility(masks_lib, lq, lk, window, causal):
    ref = visible_cells(lq, lk, window, causal)
    nkb = -(-lk // 64)
    qm = np.zeros((lq, nkb * 64), np.uint8)
    masks_lib.qm_cells(lq, lk, window, int(causal), qm.ctypes.data)
    assert np.array_equal(qm[:, :lk].astype(bool), ref)
    assert not qm[:, lk:].any(), "keys past L_k must be masked"
    nqb = -(-lq // 32)
    km = np.zeros((nqb * 32, lk), np.uint8)
    masks_lib.km_cells(lq, lk, window, int(causal), km.ctypes.data)
    assert np.array_equal(km[:lq].astype(bool), ref)
    assert not km[lq:].any(), "rows past L_q must be masked"
