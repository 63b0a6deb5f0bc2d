// Forward and backward attention kernels for gfx950, and their launchers.
//
// Forward (per block of query rows and heads of one KV group): S^T = K Q^T on
// MFMA, mask edge cells, online softmax per query in the exp2 domain, O^T +=
// V^T P^T on MFMA; the epilogue writes O and the natural-log LSE. The
// mlx-train-perf README's flash-attention passage describes this saved state
// (the output and the log-sum-exp) and the tile recompute in the backward.
//
// Backward, two launches on the caller's stream:
//   dq:    per block of query rows: D = rowsum(dO * O) and LSE * log2 e for
//          its rows (written to the workspace for dkdv), then per key tile:
//          recompute S^T, dP^T = V dO^T, P = exp(S - LSE), dS = P (dP - D),
//          dQ^T += K^T dS^T. The accumulator is cleared before the first
//          visited key tile, which under a window is not tile zero ("Off
//          NVIDIA, you fix the platform yourself", section "What did fixing
//          it take?").
//   dkdv:  per key tile of BN keys and KV head: K and V stay in LDS (fp32 and
//          head_dim 256: in registers; head_dim 256 walks the query tiles
//          twice, dV first, then dK); for each query head of the group and each query tile
//          that sees the key tile: S = Q K^T, dP = dO V^T, dV^T += dO^T P,
//          dK^T += Q^T dS. A key tile no query sees writes exact zeros (same
//          section: some key blocks are never visited).
// A separate D launch (delta) serves callers of the stage API who run dkdv
// without dq.
// Score tiles S, P, dP, dS stay fp32 in registers; P and dS are rounded to
// bf16 only as MFMA operands (the lab record's "Attention gradient error, real
// Gemma 4 activations" entry: bf16 scratch scores cost about fourfold in dQ
// error against fp32 score tiles).
//
// Every kernel streams its shared operand tiles (K/V, or Q/dO) through two LDS
// stages: the next tile's global-to-LDS loads are issued during the current
// step into the other stage and waited for at the step's one barrier.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "../../include/swa_attn.h"
#include "kernel_common.hpp"
#include "launch.hpp"
#include "sched.hpp"

namespace swa {

// Store 4 consecutive fp32 values as T (8 bytes for bf16 and fp16, 16 for fp32).
template <typename T> __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *reinterpret_cast<bf16x4*>(p) = v;
}
template <> __device__ __forceinline__ void store4<fp16>(fp16* p, float a, float b, float c, float d) {
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  f16x4 v = {(fp16)a, (fp16)b, (fp16)c, (fp16)d};
  *reinterpret_cast<f16x4*>(p) = v;
}
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}

// Write a D/32-block accumulator set (one query or key per lane, rows = head
// dim) to row pointer `row`, multiplied by `mul`.
template <typename T, int D>
__device__ __forceinline__ void store_acc_rows(T* row, const f32x16 (&acc)[D / 32], float mul, int half) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * dt + 8 * r4 + 4 * half;
      store4<T>(row + d, acc[dt][4 * r4] * mul, acc[dt][4 * r4 + 1] * mul, acc[dt][4 * r4 + 2] * mul,
                acc[dt][4 * r4 + 3] * mul);
    }
}

// Register-staged copy of one ROWS x D tile: load() issues the global reads
// (rows >= valid read as zero), store() writes the swizzled LDS stage.
template <typename T, int ROWS, int D, int NT>
struct TileStage {
  using Tile = LdsTile<T, ROWS, D>;
  static constexpr int kTotal = ROWS * Tile::kChunks;
  static constexpr int kPer = kTotal / NT;
  static_assert(kTotal % NT == 0, "tile must split evenly over the workgroup");
  u32x4 r[kPer];
  __device__ __forceinline__ void load(const T* __restrict__ src, int64_t stride, int valid, int tid) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int idx = tid + e * NT;
      const int row = idx / Tile::kChunks, c = idx % Tile::kChunks;
      r[e] = u32x4{0u, 0u, 0u, 0u};
      if (row < valid)
        r[e] = *reinterpret_cast<const u32x4*>(src + (int64_t)row * stride + c * Tile::kElemsPerChunk);
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int idx = tid + e * NT;
      const int row = idx / Tile::kChunks, c = idx % Tile::kChunks;
      *reinterpret_cast<u32x4*>(lds + Tile::chunk_off(row, c)) = r[e];
    }
  }
};

// Key tile kb of one sequence (K or V rows) into an LDS tile.
template <typename T, int BN, int D, int NT>
__device__ __forceinline__ void fill_tile(const TileLoader<T, BN, D, NT>& ld, char* dst, const T* X, int64_t kstride,
                                          int kb, int lk) {
  const int kvalid = min(BN, lk - kb * BN);
  ld.issue(dst, X + (int64_t)kb * BN * kstride, (uint32_t)(kstride * sizeof(T)), kvalid);
}
// K and V key tile kb of one sequence into an LDS stage (K tile, then V tile).
template <typename T, int BN, int D, int NT>
__device__ __forceinline__ void fill_kv(const TileLoader<T, BN, D, NT>& ld, char* st, const T* K, const T* V,
                                        int64_t kstride, int kb, int lk) {
  fill_tile(ld, st, K, kstride, kb, lk);
  fill_tile(ld, st + LdsTile<T, BN, D>::kBytes, V, kstride, kb, lk);
}

// Query-major work items (forward and dQ). A workgroup's 4 waves take HW query
// heads of one KV group (HW = 4, 2 or 1: the largest that divides the group)
// and 128 / HW query rows, 32 rows per wave. All of them read the same K/V
// tiles, and the key range the workgroup visits spans the window plus 32 or
// 64 rows instead of 128, so fewer key tiles are computed only in part (at a
// 1,024 window: 17 instead of 19 64-key tiles per 32-row wave).
__host__ __device__ inline int query_heads_per_wg(int heads_q, int heads_kv) {
  const int grp = heads_q / heads_kv;
  return grp % 4 == 0 ? 4 : (grp % 2 == 0 ? 2 : 1);
}
struct GroupedItem {
  int qb, rows, h, b, q0, lq, k0, lk, g, row0;  // row0: first row of this wave
};
// Logical order: KV head (outermost), sequence, row block (descending: under
// the causal mask later blocks see more keys, so the longest run first), head
// chunk within the group (innermost). The launch id is remapped so that each
// XCD runs a contiguous logical range.
__device__ __forceinline__ GroupedItem decode_grouped_item(const AttnArgs& a, int w) {
  GroupedItem it;
  const int hw = 1 << a.q_hw_log2;
  it.rows = a.q_rows;
  uint32_t L = (uint32_t)xcd_remap((int)blockIdx.x, a.q_items);
  uint32_t q = fast_div(L, a.div_nch);
  const int ch = (int)(L - q * (uint32_t)a.q_nch);
  L = q;
  q = fast_div(L, a.div_nqb);
  it.qb = a.q_nqb - 1 - (int)(L - q * (uint32_t)a.q_nqb);
  L = q;
  q = fast_div(L, a.div_batch);
  it.b = (int)(L - q * (uint32_t)a.batch);
  it.g = (int)q;
  it.h = it.g * a.q_grp + ch * hw + (w & (hw - 1));
  it.row0 = it.qb * it.rows + 32 * (w >> a.q_hw_log2);
  it.q0 = a.cu_q[it.b];
  it.lq = a.cu_q[it.b + 1] - it.q0;
  it.k0 = a.cu_k[it.b];
  it.lk = a.cu_k[it.b + 1] - it.k0;
  return it;
}

// ---------------------------------------------------------------- forward
// Lazy rescaling: the running reference max m moves only when a row's max
// exceeds it by more than kRescaleSlack (log2 units), so P = 2^(s*c - m) stays
// below 2^kRescaleSlack and the O accumulator is rescaled rarely. The result
// is the same softmax: O and LSE use the same reference at the end.
constexpr float kRescaleSlack = 8.0f;

// ------------------------------------------------ mask combined with the window
// Mask row t (packed query token) is a.mask_words words; bit j % 32 of word
// j / 32 allows key j of the token's sequence.

// The words of query row t that cover key tile kb of NW * 32 keys; zeros for a
// row past L_q (masked, never stored).
template <int NW>
__device__ __forceinline__ void row_mask_words(const AttnArgs& a, int64_t t, bool ok, int kb,
                                               uint32_t (&mw)[NW]) {
  static_assert(NW == 1 || NW == 2, "32- or 64-key tiles");
  if constexpr (NW == 2) {
    if (ok) {
      const uint2 v = *reinterpret_cast<const uint2*>(a.mask + t * a.mask_words + (int64_t)NW * kb);
      mw[0] = v.x;
      mw[1] = v.y;
    } else {
      mw[0] = mw[1] = 0u;
    }
  } else {
    mw[0] = ok ? a.mask[t * a.mask_words + kb] : 0u;
  }
}

// Query-major score tiles (one query per lane; element r of 32-key block kt
// is key 32 kt + 8 (r / 4) + 4 half + r % 4 of the tile): -inf where the
// query's bit for that key is clear.
__device__ __forceinline__ void apply_row_mask(f32x16& s, uint32_t word, int half) {
  const uint32_t w = word >> (4 * half);
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (!((w >> (8 * (r >> 2) + (r & 3))) & 1u)) s[r] = -INFINITY;
}
// Key-major score tiles (one key per lane, bit `bit` of each row's word;
// element r is query row 8 (r / 4) + 4 half + r % 4 of the block): -inf where
// the row's bit for the lane's key is clear. Skipped when every word the wave
// holds is all ones.
__device__ __forceinline__ void apply_col_mask(f32x16& s, const uint32_t (&words)[16], int bit) {
  uint32_t all = words[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) all &= words[r];
  if (__all(all == 0xFFFFFFFFu)) return;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (!((words[r] >> bit) & 1u)) s[r] = -INFINITY;
}
// Every block of a 32- or 64-key tile; skipped when every lane's words are
// all ones (a tile inside one document, say), which the wave decides as a
// whole.
template <int NW>
__device__ __forceinline__ void apply_row_masks(f32x16 (&s)[NW], const uint32_t (&mw)[NW], int half) {
  uint32_t all = mw[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) all &= mw[i];
  if (__all(all == 0xFFFFFFFFu)) return;
#pragma unroll
  for (int i = 0; i < NW; ++i) apply_row_mask(s[i], mw[i], half);
}

// ------------------------------------------- ranges of the mask's allowed bits
// For each sequence and each 32-row block of its queries: the first and last
// 32-key block (mask word) in which some row of the block has an allowed bit
// among the keys the window can show that block (row ranges); for each
// 32-key block of its keys: the first and last 32-row block with such a bit
// among the rows the window lets see that block (column ranges). Empty ranges
// are (1, 0). The kernels intersect their tile ranges with these, so tiles
// at a range's ends that the mask empties are never visited; a tile whose
// cells are all masked contributes nothing, so the results are unchanged.
// Words are tested whole: bits of a word the window partly hides still count,
// which can only widen a range. One wave per block: the first `nrb_total`
// waves take row blocks, the rest key blocks.
__global__ void __launch_bounds__(64) mask_range_kernel(AttnArgs a, int32_t* ranges, int nrb, int nkb32) {
  const int lane = threadIdx.x;
  const int64_t nrows = (int64_t)a.batch * nrb;
  int64_t id = blockIdx.x;
  const bool rows = id < nrows;
  if (!rows) id -= nrows;
  const int per = rows ? nrb : nkb32;
  const int b = (int)(id / per), blk = (int)(id % per);
  const int q0 = a.cu_q[b], lq = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], lk = a.cu_k[b + 1] - k0;
  const SeqGeom sg{lq, lk, a.window, a.causal != 0};
  int first = INT32_MAX, last = -1;
  if (rows) {
    // keys the window shows rows [32 blk, 32 blk + 31]
    const TileRange kr = query_tile_keys(sg, blk, 32, 32);
    const int i = 32 * blk + (lane & 31);
    if (i < lq)
      for (int w = kr.lo + (lane >> 5); w <= kr.hi; w += 2)
        if (a.mask[(int64_t)(q0 + i) * a.mask_words + w] != 0u) {
          first = min(first, w);
          last = max(last, w);
        }
  } else {
    // rows the window lets see keys [32 blk, 32 blk + 31]
    const TileRange qr = key_tile_queries(sg, blk, 32, 1);
    for (int i = qr.lo + lane; i <= qr.hi; i += 64)
      if (a.mask[(int64_t)(q0 + i) * a.mask_words + blk] != 0u) {
        first = min(first, i >> 5);
        last = max(last, i >> 5);
      }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    first = min(first, __shfl_xor(first, off, 64));
    last = max(last, __shfl_xor(last, off, 64));
  }
  if (lane == 0) {
    int32_t* r = ranges + 2 * ((rows ? 0 : nrows) + id);
    r[0] = last >= 0 ? first : 1;
    r[1] = last >= 0 ? last : 0;
  }
}

// The union of the ranges of blocks [blk0, blk0 + nblk) (row or key blocks of
// sequence b, `row` picks which table), in units of `unit` 32-blocks,
// intersected with [lo, hi]. Returns an empty range (lo > hi) when no block
// has an allowed bit.
__device__ __forceinline__ void narrow_by_mask(const AttnArgs& a, bool row, int b, int blk0, int nblk, int unit,
                                               int32_t& lo, int32_t& hi) {
  const int nrb = (a.max_seqlen_q + 31) / 32, nkb32 = (a.max_seqlen_k + 31) / 32;
  const int per = row ? nrb : nkb32;
  const int32_t* r = a.mask_ranges + 2 * ((row ? 0 : (int64_t)a.batch * nrb) + (int64_t)b * per);
  int first = INT32_MAX, last = -1;
  for (int k = blk0; k < blk0 + nblk && k < per; ++k) {
    const int f = r[2 * k], l = r[2 * k + 1];
    if (f <= l) {
      first = min(first, f);
      last = max(last, l);
    }
  }
  if (last < 0) {
    lo = 0;
    hi = -1;
    return;
  }
  lo = max(lo, first / unit);
  hi = min(hi, last / unit);
}

template <int N> using ic = std::integral_constant<int, N>;

// Per-query visibility as one unsigned range test with a wave-uniform limit:
// key j is visible to the query at key position p iff
// (unsigned)(mpos - j) < mlim, i.e. j lies in [mpos - mlim + 1, mpos].
// Causal: mpos = p, mlim = w. Full attention: mpos = L_k - 1, mlim = 2^31 - 1.
// Two-sided (the C ABI limits L_q and L_k to 2^30 so that mpos = p + w - 1
// fits): mlim = 2w - 1, and keys at or past L_k (the padding rows of a
// sequence's last tile) must be masked as well (pad_keys). A two-sided window
// is full attention only when w >= max(L_q, L_k): the positions run from
// L_k - L_q to L_k - 1, so with more queries than keys (p < 0 for the first
// rows) |p - j| reaches L_q - 1. A p below zero wraps mpos past every limit
// when no key is in reach. Only mpos is per lane, so the limit stays in a
// scalar register.
struct RowWindow {
  uint32_t mpos, mlim;
  bool pad_keys;
};
__device__ __forceinline__ RowWindow row_window(int p, int lq, int lk, int window, bool causal) {
  if (causal) return {(uint32_t)p, (uint32_t)window, false};
  if (window >= max(lq, lk)) return {(uint32_t)(lk - 1), 0x7fffffffu, false};
  return {(uint32_t)p + (uint32_t)(window - 1), 2u * (uint32_t)window - 1u, true};
}

// The same rule per (query position p, key j) pair for the key-major kernels,
// where registers run over queries: masked iff windowed and
// (unsigned)(p - j + off) >= lim. Causal: off 0, lim w. Two-sided
// (w < max(L_q, L_k), as above): off w - 1, lim 2w - 1. Full attention: not
// windowed.
struct PairWindow {
  bool windowed;
  int off;
  uint32_t lim;
};
__device__ __forceinline__ PairWindow pair_window(int lq, int lk, int window, bool causal) {
  if (causal) return {true, 0, (uint32_t)window};
  if (window >= max(lq, lk)) return {false, 0, 0u};
  return {true, window - 1, 2u * (uint32_t)window - 1u};
}

// Edge-tile masks as bit runs. Within one tile the visible cells of a lane's
// row (or, key-major, of a lane's key) form one interval of offsets, so the
// mask is one run of ones, built once per tile; each cell then costs a
// sign-extended bit field and a bit select instead of compares.
__device__ __forceinline__ uint64_t bit_run(int lo, int hi) {  // bits [lo, hi), 0 <= lo, hi <= 64
  if (hi <= lo) return 0ull;
  return (hi >= 64 ? ~0ull : (1ull << hi) - 1ull) & ~((1ull << lo) - 1ull);
}
// Query-major: bit o set iff (unsigned)(mb - o) < mlim (row_window, with mb =
// mpos - the key of offset 0) and, with nk >= 0, o < nk (keys past L_k).
// Offsets past mb wrap to at least 2^32 - 64 > mlim, so they are never visible.
__device__ __forceinline__ uint64_t row_keys_visible(uint32_t mb, uint32_t mlim, int nk) {
  const int hi = (int)min(mb, 63u) + 1;
  const int lo = mb >= mlim ? (int)min(mb - mlim + 1u, 64u) : 0;
  return bit_run(lo, nk >= 0 ? min(hi, nk) : hi);
}
// Key-major: bit o set iff row ib + o is a real row (< L_q) and, when
// windowed, (unsigned)(mb + o) < lim (pair_window, mb = ib + L_k - L_q - j +
// off). Two-sided windows need L_q, L_k <= 2^30 (the C ABI's limit), so
// |p - j| and off stay below 2^30; causal ones have off = 0 and |p - j| below
// the longer length plus 32: mb and the bounds stay in int range.
__device__ __forceinline__ uint32_t key_rows_visible(int ib, int mb, int lq, const PairWindow& pw) {
  int hi = min(max(lq - ib, 0), 32), lo = 0;
  if (pw.windowed) {
    const int lim = (int)pw.lim;
    lo = min(max(-mb, 0), 32);
    hi = min(hi, mb >= lim ? 0 : (mb < lim - 32 ? 32 : lim - mb));
  }
  return (uint32_t)bit_run(lo, hi);
}
// s[r] (offset o = 8 (r / 4) + r % 4 in the lane's 32-cell block) becomes -inf
// where bit o of vis is clear
__device__ __forceinline__ void apply_visible(f32x16& s, uint32_t vis) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int o = 8 * (r >> 2) + (r & 3);
    const int keep = (int)(vis << (31 - o)) >> 31;
    s[r] = __int_as_float((__float_as_int(s[r]) & keep) | (~keep & (int)0xff800000u));
  }
}

// Waves per SIMD of the query-major kernels: two for 16-bit types up to
// head_dim 128 (256 registers each; one wave's softmax overlaps the other's
// MFMAs); one at head_dim 256 and for fp32 at 128, whose accumulator and Q
// fragments need the 512-register budget (their 128 KB of K/V stages leave
// room for one workgroup per CU anyway).
template <typename T> constexpr int waves_per_simd(int d) { return d > 128 || (sizeof(T) == 4 && d > 64) ? 1 : 2; }

template <typename T, int D, int BM, int BN, bool M>
__global__ void __launch_bounds__(BM * 2) __attribute__((amdgpu_waves_per_eu(waves_per_simd<T>(D), waves_per_simd<T>(D))))
fwd_kernel(AttnArgs a) {
  static_assert(BN == 64 || (BN == 32 && D > 256), "64-key tiles (32 at head_dim 512)");
  constexpr int NT = BM * 2;
  constexpr bool kPipe = sizeof(T) == 2 && D <= 128;  // software-pipelined loop (see below)
  using KTile = LdsTile<T, BN, D>;
  // two stages (K tile then V tile each), separate arrays so that reading one
  // need not wait for the asynchronous fill of the other
  __shared__ __attribute__((aligned(1024))) char st0[2 * KTile::kBytes];
  __shared__ __attribute__((aligned(1024))) char st1[2 * KTile::kBytes];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int w = wave_uniform(tid >> 6);
  const GroupedItem it = decode_grouped_item(a, w);
  if (it.qb * it.rows >= it.lq) return;
  const int g = it.g;
  const SeqGeom sg{it.lq, it.lk, a.window, a.causal != 0};
  TileRange kr = query_tile_keys(sg, it.qb, it.rows, BN);
  // with the mask's ranges: only key tiles in which some row of the tile has
  // an allowed bit
  if constexpr (M)
    if (a.mask_ranges != nullptr) narrow_by_mask(a, true, it.b, it.qb * it.rows / 32, it.rows / 32, BN / 32, kr.lo, kr.hi);

  const int64_t qstride = (int64_t)a.heads_q * D;
  const int64_t kstride = (int64_t)a.heads_kv * D;
  const T* __restrict__ Q = static_cast<const T*>(a.q);
  const T* __restrict__ K = static_cast<const T*>(a.k) + (int64_t)it.k0 * kstride + g * D;
  const T* __restrict__ V = static_cast<const T*>(a.v) + (int64_t)it.k0 * kstride + g * D;

  const int i = it.row0 + l32;  // this lane's query row
  const bool row_ok = i < it.lq;
  const int64_t mrow = it.q0 + (row_ok ? i : 0);  // its mask row (with M)
  Frag<T> qf[D / 16];
  {
    const T* qrow = Q + (int64_t)(it.q0 + (row_ok ? i : 0)) * qstride + it.h * D + 8 * half;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = row_ok ? global_frag<T>(qrow + 16 * s) : zero_frag<T>();
  }
  RowReader<T, D> rrd;
  rrd.init(l32, half);
  ColReader<T, D> crd;
  crd.init(lane);
  // Edge mask: visible iff (unsigned)(mpos - j) < mlim (row_window). Key rows
  // past L_k in the last tile arrive as zeros and are always masked.
  const RowWindow rw = row_window(i + (it.lk - it.lq), it.lq, it.lk, a.window, a.causal != 0);
  const uint32_t mpos = rw.mpos, mlim = rw.mlim;

  const float c = a.scale * kLog2e;
  // O = acc / l (columns col0 ..), LSE = m + log2(l) in natural log
  auto finish = [&](auto& acc_, float m_, float lsum_, int col0, bool with_lse) __attribute__((always_inline)) {
    constexpr int DW = 32 * (int)(sizeof(acc_) / sizeof(acc_[0]));
    const float ltot = sum_halves(lsum_);
    if (row_ok) {
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
      T* orow = static_cast<T*>(a.out_o) + (int64_t)(it.q0 + i) * qstride + it.h * D + col0;
      store_acc_rows<T, DW>(orow, acc_, inv, half);
      if (with_lse && half == 0)
        a.out_lse[(int64_t)it.h * a.total_q + it.q0 + i] =
            ltot > 0.f ? (m_ + fast_log2(ltot)) * kLn2 : -INFINITY;
    }
  };

  TileLoader<T, BN, D, NT> kvld;
  kvld.init((uint32_t)(kstride * sizeof(T)), w, lane);
  // an odd number of tiles starts in stage 1, so that the loop below runs
  // whole (stage 0, stage 1) pairs: with no exit between the two steps the
  // accumulators keep their registers across the loop (no copies)
  const int ntiles = kr.hi - kr.lo + 1;
  if constexpr (kPipe) {
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
    float m = -INFINITY, lsum = 0.f;
    // Software pipeline over key tiles: step j puts tile j+1's scores on the
    // MFMA unit while the VALU turns tile j's scores into probabilities, then
    // adds tile j's P V. K and V tiles rotate through their own two stages:
    // K_{j+2} and V_{j+1} load during step j. Tile j sits in stage (j + p) & 1
    // with p = (ntiles - 1) & 1, so the loop runs whole stage pairs and the
    // last tile, which has no successor, is in stage 0.
    const int p = (ntiles - 1) & 1;
    if (ntiles > 0) {
      fill_kv(kvld, p ? st1 : st0, K, V, kstride, kr.lo, it.lk);
      if (ntiles > 1) fill_tile(kvld, p ? st0 : st1, K, kstride, kr.lo + 1, it.lk);
    }
    __syncthreads();
    auto qk = [&](f32x16 (&s)[BN / 32], const char* ks) __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt) {
        s[kt] = f32x16{};
#pragma unroll
        for (int ss = 0; ss < D / 16; ++ss) mma(s[kt], rrd.read(ks, 32 * kt, ss), qf[ss]);
      }
    };
    // one step: tile kb's scores in `cur` (K and V in stage `stage`); with a
    // successor, its scores go to `nxt` from the other stage's K tile
    // With M, the mask words of tile kb are in `mcur`; the next tile's load into `mnxt`.
    auto pstep = [&](auto stage_c, auto next_c, int kb, f32x16 (&cur)[BN / 32], f32x16 (&nxt)[BN / 32],
                     uint32_t (&mcur)[BN / 32], uint32_t (&mnxt)[BN / 32]) __attribute__((always_inline)) {
      constexpr int stage = decltype(stage_c)::value;
      constexpr bool has_next = decltype(next_c)::value;
      char* here = stage ? st1 : st0;
      char* other = stage ? st0 : st1;
      if constexpr (has_next) {
        if (kb + 2 <= kr.hi) fill_tile(kvld, here, K, kstride, kb + 2, it.lk);
        fill_tile(kvld, other + KTile::kBytes, V, kstride, kb + 1, it.lk);
        if constexpr (M) row_mask_words(a, mrow, row_ok, kb + 1, mnxt);
      }
      if (!(kr.full_lo <= kb && kb <= kr.full_hi)) {  // edge tile: mask cell by cell
        const int jb = kb * BN + 4 * half;  // two-sided: the keys past L_k are masked as well
        const uint64_t vis = row_keys_visible(mpos - (uint32_t)jb, mlim, rw.pad_keys ? max(it.lk - jb, 0) : -1);
#pragma unroll
        for (int kt = 0; kt < BN / 32; ++kt) apply_visible(cur[kt], (uint32_t)(vis >> (32 * kt)));
      }
      if constexpr (M) apply_row_masks(cur, mcur, half);
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, cur[kt][r]);
      mx = max_halves(mx);
      const float mxs = mx == -INFINITY ? -INFINITY : mx * c;
      const bool grow = mxs > m + kRescaleSlack;
      if (__any(grow)) {
        const float mnew = grow ? mxs : m;
        const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mnew);
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;
        m = mnew;
      }
      if constexpr (has_next) qk(nxt, other);
      const float mu = m == -INFINITY ? 0.f : m;
      Frag<T> pf[BN / 16];
      float rs = 0.f;
#pragma unroll
      for (int u = 0; u < BN / 16; ++u) {
        f32x16& sv = cur[u >> 1];
#pragma unroll
        for (int r = 8 * (u & 1); r < 8 * (u & 1) + 8; ++r) sv[r] = fast_exp2(fmaf(sv[r], c, -mu));
        pf[u] = acc_frag<T>(sv, u & 1);
        rs = frag_sum(pf[u], rs);  // over the rounded P that the MFMA multiplies
      }
      lsum += rs;
#pragma unroll
      for (int u = 0; u < BN / 16; ++u)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) mma(acc[dt], crd.read(here + KTile::kBytes, 16 * u, dt), pf[u]);
      if constexpr (has_next) __syncthreads();
    };
    if (ntiles > 0) {
      f32x16 sa[BN / 32], sb[BN / 32];
      uint32_t ma[BN / 32] = {}, mb[BN / 32] = {};
      int kb = kr.lo;
      // the first step refills the first tile's K stage: every wave must have
      // read it first (later steps meet a barrier between the two)
      if (p) {
        if constexpr (M) row_mask_words(a, mrow, row_ok, kb, mb);
        qk(sb, st1);
        __syncthreads();
        pstep(ic<1>{}, std::true_type{}, kb++, sb, sa, mb, ma);
      } else {
        if constexpr (M) row_mask_words(a, mrow, row_ok, kb, ma);
        qk(sa, st0);
        __syncthreads();
      }
      for (; kb < kr.hi; kb += 2) {
        pstep(ic<0>{}, std::true_type{}, kb, sa, sb, ma, mb);
        pstep(ic<1>{}, std::true_type{}, kb + 1, sb, sa, mb, ma);
      }
      pstep(ic<0>{}, std::false_type{}, kb, sa, sb, ma, mb);
    }
    finish(acc, m, lsum, 0, true);
  } else {
  // O columns per pass over the key tiles: all of them up to head_dim 256; at
  // 512 four passes of 128 (the accumulator and the Q fragments together would
  // exceed the registers of one wave), each recomputing S and the softmax
  // statistics exactly as the others do
  constexpr int DO = D > 256 ? 128 : D;
#pragma unroll 1
  for (int pass = 0; pass < D / DO; ++pass) {
  f32x16 acc[DO / 32];
#pragma unroll
  for (int dt = 0; dt < DO / 32; ++dt) acc[dt] = f32x16{};
  float m = -INFINITY, lsum = 0.f;
  if (ntiles > 0) {
    if (ntiles & 1) fill_kv(kvld, st1, K, V, kstride, kr.lo, it.lk);
    else fill_kv(kvld, st0, K, V, kstride, kr.lo, it.lk);
  }
  __syncthreads();

  // One key tile; `stage` (compile time) selects the LDS stage it reads.
  auto step = [&](auto stage_c, int kb) {
    constexpr int stage = decltype(stage_c)::value;
    const char* ks = stage ? st1 : st0;
    const char* vs = ks + KTile::kBytes;
    if (kb < kr.hi) fill_kv(kvld, stage ? st0 : st1, K, V, kstride, kb + 1, it.lk);
    // Edge tiles are masked cell by cell. A wave whose 32 rows see none of an
    // edge tile's keys still computes it (P = 0): an early exit from the step
    // makes the compiler copy the O accumulator at every step, which costs more
    // than the few all-masked wave tiles.
    const bool edge = !(kr.full_lo <= kb && kb <= kr.full_hi);
    uint32_t mw[BN / 32] = {};
    if constexpr (M) row_mask_words(a, mrow, row_ok, kb, mw);
    f32x16 s[BN / 32];
#pragma unroll
    for (int kt = 0; kt < BN / 32; ++kt) {
      s[kt] = f32x16{};
#pragma unroll
      for (int ss = 0; ss < D / 16; ++ss) mma(s[kt], rrd.read(ks, 32 * kt, ss), qf[ss]);
    }
    if (edge) {  // two-sided: the keys past L_k are masked as well
      const int k0l = kb * BN + 4 * half;
      const uint64_t vis = row_keys_visible(mpos - (uint32_t)k0l, mlim, rw.pad_keys ? max(it.lk - k0l, 0) : -1);
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt) apply_visible(s[kt], (uint32_t)(vis >> (32 * kt)));
    }
    if constexpr (M) apply_row_masks(s, mw, half);
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = max_halves(mx);
    const float mxs = mx == -INFINITY ? -INFINITY : mx * c;
    const bool grow = mxs > m + kRescaleSlack;
    if (__any(grow)) {
      const float mnew = grow ? mxs : m;
      const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DO / 32; ++dt) acc[dt] *= alpha;
      m = mnew;
    }
    const float mu = m == -INFINITY ? 0.f : m;
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(fmaf(s[kt][r], c, -mu));
        s[kt][r] = pv;
        if constexpr (sizeof(T) == 4) rs += pv;
      }
    // bf16: the row sum is taken over the rounded P that the MFMA multiplies,
    // so O's weights sum to exactly the normaliser
#pragma unroll
    for (int u = 0; u < BN / 16; ++u) {
      const Frag<T> pf = acc_frag<T>(s[u >> 1], u & 1);
      if constexpr (sizeof(T) == 2) rs = frag_sum(pf, rs);
#pragma unroll
      for (int dt = 0; dt < DO / 32; ++dt) mma(acc[dt], crd.read(vs, 16 * u, pass * (DO / 32) + dt), pf);
    }
    lsum += rs;
    __syncthreads();
  };
  int kb = kr.lo;
  if (ntiles & 1) step(ic<1>{}, kb++);
  for (; kb <= kr.hi; kb += 2) {
    step(ic<0>{}, kb);
    step(ic<1>{}, kb + 1);
  }
  finish(acc, m, lsum, pass * DO, pass == 0);
  }
  }
}

// ------------------------------------------ backward: D = rowsum(dO*O), LSE*log2e
// The second output lets the other backward kernels copy LSE into LDS raw:
// P = 2^(S * scale * log2e - LSE * log2e); a row without visible keys
// (LSE = -inf) gets +inf, so its P is 0.
// A block takes one query head and kDeltaPasses x (256 / LPR) consecutive
// tokens; in each pass LPR lanes share a (token, head) row, 8 elements per
// lane, and the rows of a pass are consecutive tokens of the head, so their D
// and LSE*log2e land in consecutive words of the [Hq, T] outputs. All of a
// thread's loads are issued before the first reduction.
constexpr int kDeltaPasses = 4;
template <int D> constexpr int delta_tokens_per_block() { return kDeltaPasses * (256 / (D / 8)); }
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_delta_kernel(AttnArgs a) {
  constexpr int LPR = D / 8;  // lanes per (token, head) row, 8 elements each
  constexpr int RPP = 256 / LPR;
  constexpr int TPB = delta_tokens_per_block<D>();
  const int h = (int)(blockIdx.x % (unsigned)a.heads_q);
  const int64_t t0 = (int64_t)(blockIdx.x / (unsigned)a.heads_q) * TPB;
  const int sub = threadIdx.x % LPR, rs = threadIdx.x / LPR;
  Frag<T> o[kDeltaPasses], d[kDeltaPasses];
#pragma unroll
  for (int p = 0; p < kDeltaPasses; ++p) {
    const int64_t t = t0 + p * RPP + rs;
    if (t < a.total_q) {
      const int64_t off = (t * a.heads_q + h) * D + sub * 8;
      o[p] = global_frag<T>(static_cast<const T*>(a.o) + off);
      d[p] = global_frag<T>(static_cast<const T*>(a.dout) + off);
    } else {
      o[p] = zero_frag<T>();
      d[p] = zero_frag<T>();
    }
  }
#pragma unroll
  for (int p = 0; p < kDeltaPasses; ++p) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += to_f32(o[p].v[j]) * to_f32(d[p].v[j]);
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    const int64_t t = t0 + p * RPP + rs;
    if (sub == 0 && t < a.total_q) {
      const int64_t idx = (int64_t)h * a.total_q + t;
      a.delta[idx] = -acc;
      const float l = a.lse[idx];
      a.lse2[idx] = l == -INFINITY ? INFINITY : l * kLog2e;
    }
  }
}

// ------------------------------------------------------------- backward: dQ
template <typename T, int D, int BM, int BN, bool M>
__global__ void __launch_bounds__(BM * 2) __attribute__((amdgpu_waves_per_eu(waves_per_simd<T>(D), waves_per_simd<T>(D))))
bwd_dq_kernel(AttnArgs a) {
  static_assert(BN == 64 || (BN == 32 && D > 256), "64-key tiles (32 at head_dim 512)");
  // dQ columns accumulated per pass over the key tiles: all of them up to
  // head_dim 256; at 512 four passes of 128 (the accumulator, Q and dO
  // fragments together would exceed the registers of one wave), each
  // recomputing S and dP
  constexpr int DO = D > 256 ? 128 : D;
  constexpr int NT = BM * 2;
  using KTile = LdsTile<T, BN, D>;
  __shared__ __attribute__((aligned(1024))) char st0[2 * KTile::kBytes];
  __shared__ __attribute__((aligned(1024))) char st1[2 * KTile::kBytes];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int w = wave_uniform(tid >> 6);
  const GroupedItem it = decode_grouped_item(a, w);
  if (it.qb * it.rows >= it.lq) return;
  const int g = it.g;
  const SeqGeom sg{it.lq, it.lk, a.window, a.causal != 0};
  TileRange kr = query_tile_keys(sg, it.qb, it.rows, BN);
  // with the mask's ranges: only key tiles in which some row of the tile has
  // an allowed bit
  if constexpr (M)
    if (a.mask_ranges != nullptr) narrow_by_mask(a, true, it.b, it.qb * it.rows / 32, it.rows / 32, BN / 32, kr.lo, kr.hi);

  const int64_t qstride = (int64_t)a.heads_q * D;
  const int64_t kstride = (int64_t)a.heads_kv * D;
  const T* __restrict__ K = static_cast<const T*>(a.k) + (int64_t)it.k0 * kstride + g * D;
  const T* __restrict__ V = static_cast<const T*>(a.v) + (int64_t)it.k0 * kstride + g * D;

  const int i = it.row0 + l32;
  const bool row_ok = i < it.lq;
  const int64_t mrow = it.q0 + (row_ok ? i : 0);  // its mask row (with M)
  Frag<T> qf[D / 16], df[D / 16];
  float lse2 = INFINITY, dlt = 0.f;
  {
    const int64_t roff = (int64_t)(it.q0 + (row_ok ? i : 0)) * qstride + it.h * D + 8 * half;
    const T* qrow = static_cast<const T*>(a.q) + roff;
    const T* drow = static_cast<const T*>(a.dout) + roff;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qf[s] = row_ok ? global_frag<T>(qrow + 16 * s) : zero_frag<T>();
      df[s] = row_ok ? global_frag<T>(drow + 16 * s) : zero_frag<T>();
    }
    // D = rowsum(dO * O) for this row: this lane holds half of each 16-dim
    // chunk of dO (df) and reads the same half of O; the two lane halves' sums
    // are added across the wave
    const T* orow = static_cast<const T*>(a.o) + roff;
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const Frag<T> of = row_ok ? global_frag<T>(orow + 16 * s) : zero_frag<T>();
#pragma unroll
      for (int j = 0; j < 8; ++j) part = fmaf(to_f32(of.v[j]), to_f32(df[s].v[j]), part);
    }
    dlt = sum_halves(part);
    if (row_ok) {
      const int64_t idx = (int64_t)it.h * a.total_q + it.q0 + i;
      const float l = a.lse[idx];
      lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
      if (half == 0) {
        a.delta[idx] = -dlt;
        a.lse2[idx] = lse2;
      }
    }
  }
  // dP - D: every dP accumulator starts at -D (this lane's row) instead of 0,
  // so dS = P * dP needs no subtraction per cell
  f32x16 ndlt;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndlt[r] = -dlt;
  RowReader<T, D> rrd;
  rrd.init(l32, half);
  ColReader<T, D> crd;
  crd.init(lane);
  const RowWindow rw = row_window(i + (it.lk - it.lq), it.lq, it.lk, a.window, a.causal != 0);
  const uint32_t mpos = rw.mpos, mlim = rw.mlim;
  const float c = a.scale * kLog2e;

  TileLoader<T, BN, D, NT> kvld;
  kvld.init((uint32_t)(kstride * sizeof(T)), w, lane);
  const int ntiles = kr.hi - kr.lo + 1;
#pragma unroll 1
  for (int pass = 0; pass < D / DO; ++pass) {
  // cleared before the first visited key tile (kr.lo), not on key tile zero
  f32x16 acc[DO / 32];
#pragma unroll
  for (int dt = 0; dt < DO / 32; ++dt) acc[dt] = f32x16{};
  // an odd number of tiles starts in stage 1, so that the loop below runs
  // whole (stage 0, stage 1) pairs: with no exit between the two steps the
  // accumulators keep their registers across the loop (no copies)
  if (ntiles > 0) {
    if (ntiles & 1) fill_kv(kvld, st1, K, V, kstride, kr.lo, it.lk);
    else fill_kv(kvld, st0, K, V, kstride, kr.lo, it.lk);
  }
  __syncthreads();

  auto step = [&](auto stage_c, int kb) {
    constexpr int stage = decltype(stage_c)::value;
    const char* ks = stage ? st1 : st0;
    const char* vs = ks + KTile::kBytes;
    if (kb < kr.hi) fill_kv(kvld, stage ? st0 : st1, K, V, kstride, kb + 1, it.lk);
    // Edge tiles are masked cell by cell; a wave's all-masked 32 x 64 block is
    // computed like any other (P = dS = 0): an early exit from the step made
    // the compiler copy the accumulators at every step and spill, which cost
    // more (6% of dQ) than the few all-masked blocks.
    const bool edge = !(kr.full_lo <= kb && kb <= kr.full_hi);
    uint32_t mw[BN / 32] = {};
    if constexpr (M) row_mask_words(a, mrow, row_ok, kb, mw);
    // the edge mask and (with M) the caller's mask on key block kt's scores
    auto mask_block = [&](f32x16& s, int kt) __attribute__((always_inline)) {
      if (edge) {
        const int jb = kb * BN + 32 * kt + 4 * half;  // two-sided: the keys past L_k are masked as well
        uint32_t vis = (uint32_t)row_keys_visible(mpos - (uint32_t)jb, mlim, rw.pad_keys ? max(it.lk - jb, 0) : -1);
        // at head_dim 512 the Q and dO fragments alone take 256 registers; the
        // compiler hoisted a tile's 16 per-cell masks out of the key loop and
        // spilled them (16 scratch reloads per edge tile). An empty asm
        // statement that claims to change vis keeps them here.
        if constexpr (D > 256) asm volatile("" : "+v"(vis));
        apply_visible(s, vis);
      }
      // the mask test is skipped when the whole wave's words for this block are all ones
      if constexpr (M) {
        if (!__all(mw[kt] == 0xFFFFFFFFu)) apply_row_mask(s, mw[kt], half);
      }
    };
    if constexpr (BN / 32 == 2 && D > 128) {
      // One wave per SIMD (head_dim 256): no second wave's MFMAs hide the
      // softmax, so this wave overlaps it with its own MFMAs. Key block 1's S
      // and dP MFMAs issue with block 0's softmax between them, and the dQ
      // MFMAs of block 0 with block 1's softmax between them; scheduling
      // fences keep that order, and each chunk reads the next chunk's
      // operands first. (At head_dim 128, where two waves share a SIMD, the
      // same measured within 1% either way.)
      f32x16 s0 = f32x16{}, dp0 = ndlt, s1 = f32x16{}, dp1 = ndlt;
#pragma unroll
      for (int ss = 0; ss < D / 16; ++ss) {
        mma(s0, rrd.read(ks, 0, ss), qf[ss]);
        mma(dp0, rrd.read(vs, 0, ss), df[ss]);
      }
      mask_block(s0, 0);
      {
        Frag<T> x0 = rrd.read(ks, 32, 0), y0 = rrd.read(vs, 32, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ss = 0; ss < D / 16; ++ss) {
          Frag<T> x1 = x0, y1 = y0;
          if (ss + 1 < D / 16) {
            x1 = rrd.read(ks, 32, ss + 1);
            y1 = rrd.read(vs, 32, ss + 1);
          }
          mma(s1, x0, qf[ss]);
          mma(dp1, y0, df[ss]);
#pragma unroll
          for (int e2 = 0; e2 < 16 / (D / 16); ++e2) {
            const int r = (16 / (D / 16)) * ss + e2;
            const float pv = fast_exp2(fmaf(s0[r], c, -lse2));
            s0[r] = pv * dp0[r];
          }
          __builtin_amdgcn_sched_barrier(0);
          x0 = x1;
          y0 = y1;
        }
      }
      mask_block(s1, 1);
      {
        const Frag<T> d00 = acc_frag<T>(s0, 0), d01 = acc_frag<T>(s0, 1);
        Frag<T> z0 = crd.read(ks, 0, pass * (DO / 32));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 2 * (DO / 32); ++k) {
          const int u = k / (DO / 32), dt = k % (DO / 32);
          Frag<T> z1 = z0;
          if (k + 1 < 2 * (DO / 32)) {
            const int u1 = (k + 1) / (DO / 32), dt1 = (k + 1) % (DO / 32);
            z1 = crd.read(ks, 16 * u1, pass * (DO / 32) + dt1);
          }
          mma(acc[dt], z0, u ? d01 : d00);
#pragma unroll
          for (int e2 = 0; e2 < 16 / (2 * (DO / 32)); ++e2) {
            const int r = (16 / (2 * (DO / 32))) * k + e2;
            const float pv = fast_exp2(fmaf(s1[r], c, -lse2));
            s1[r] = pv * dp1[r];
          }
          __builtin_amdgcn_sched_barrier(0);
          z0 = z1;
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const Frag<T> dsf = acc_frag<T>(s1, u);
#pragma unroll
        for (int dt = 0; dt < DO / 32; ++dt) mma(acc[dt], crd.read(ks, 32 + 16 * u, pass * (DO / 32) + dt), dsf);
      }
    } else
#pragma unroll
    for (int kt = 0; kt < BN / 32; ++kt) {
      f32x16 s = f32x16{}, dp = ndlt;
#pragma unroll
      for (int ss = 0; ss < D / 16; ++ss) {
        mma(s, rrd.read(ks, 32 * kt, ss), qf[ss]);
        mma(dp, rrd.read(vs, 32 * kt, ss), df[ss]);
      }
      mask_block(s, kt);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(fmaf(s[r], c, -lse2));
        s[r] = pv * dp[r];  // dS = P (dP - D)
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const Frag<T> dsf = acc_frag<T>(s, u);
#pragma unroll
        for (int dt = 0; dt < DO / 32; ++dt) mma(acc[dt], crd.read(ks, 32 * kt + 16 * u, pass * (DO / 32) + dt), dsf);
      }
    }
    __syncthreads();
  };
  int kb = kr.lo;
  if (ntiles & 1) step(ic<1>{}, kb++);
  for (; kb <= kr.hi; kb += 2) {
    step(ic<0>{}, kb);
    step(ic<1>{}, kb + 1);
  }
  if (row_ok) {
    T* row = static_cast<T*>(a.dq) + (int64_t)(it.q0 + i) * qstride + it.h * D + pass * DO;
    store_acc_rows<T, DO>(row, acc, a.scale, half);
  }
  }
}

// fp32 accumulator blocks through LDS in their register layout: element r of
// block dt of lane l at float index l + 64 (16 dt + r)
template <int NB>
__device__ __forceinline__ void hand_over(float* red, const f32x16 (&acc)[NB], int lane) {
#pragma unroll
  for (int dt = 0; dt < NB; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[lane + (dt * 16 + r) * 64] = acc[dt][r];
}
template <int NB>
__device__ __forceinline__ void take_over(const float* red, f32x16 (&acc)[NB], int lane) {
#pragma unroll
  for (int dt = 0; dt < NB; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] += red[lane + (dt * 16 + r) * 64];
}

// ---------------------------------------------------------- backward: dK, dV
// One workgroup per (KV head, sequence, key tile of BN = 128 keys), 8 waves:
// wave w owns keys 32*(w%4) .. +31 and, in every BM = 64-row query step, the
// query rows 32*(w/4) .. +31. K and V sit in LDS once per workgroup (the B
// operands of S = Q K^T and dP = dO V^T), so the dK/dV accumulators fit beside
// everything else at two waves per SIMD. The two query halves' partial dK/dV
// are summed through LDS at the end.
// Key-major decode: KV head outermost, then sequence, then key tile ascending
// (for the causal mask early key tiles are seen by the most queries).
template <typename T, int D, int BN, int BM, bool M>
__global__ void __launch_bounds__(BN * 4) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_kernel(AttnArgs a) {
  constexpr int NT = BN * 4;  // 8 waves for BN = 128
  static_assert(BN == 128 && BM == 64, "wave layout assumes 4 key blocks x 2 query halves");
  using QTile = LdsTile<T, BM, D>;
  using KTile = LdsTile<T, BN, D>;
  // with M, the step's mask tile follows: BM rows x 16 bytes (the 4 words of
  // this key tile's 128 keys)
  constexpr int kMaskOff = 2 * QTile::kBytes + 2 * BM * 4;
  constexpr int kStage = kMaskOff + (M ? BM * 16 : 0);  // Q, dO, LSE*log2e, D[, mask]
  constexpr int kRedBlock = 32 * D * 4;                   // fp32 partial of one 32-key block
  static_assert(KTile::kBytes >= 2 * kRedBlock && kStage >= 2 * kRedBlock, "reduction reuse");
  __shared__ __attribute__((aligned(1024))) char st0[kStage];
  __shared__ __attribute__((aligned(1024))) char st1[kStage];
  __shared__ __attribute__((aligned(1024))) char klds[KTile::kBytes];
  __shared__ __attribute__((aligned(1024))) char vlds[KTile::kBytes];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int w = wave_uniform(tid >> 6);
  const int kt = w & 3, mh = w >> 2;
  static_assert(BN == 128, "the launch-id decode counts 128-key tiles (AttnArgs::k_nkb)");
  // work item: (KV head, sequence, key tile, part of the group's query heads),
  // the part innermost so that the parts of one key tile share an L2
  uint32_t L = (uint32_t)xcd_remap((int)blockIdx.x, a.k_items);
  uint32_t qt = fast_div(L, a.div_split);
  const int part = (int)(L - qt * (uint32_t)a.kv_split);
  L = qt;
  qt = fast_div(L, a.div_nkb);
  const int kb = (int)(L - qt * (uint32_t)a.k_nkb);
  L = qt;
  qt = fast_div(L, a.div_batch);
  const int b = (int)(L - qt * (uint32_t)a.batch);
  const int g = (int)qt;
  const int q0 = a.cu_q[b], lq = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], lk = a.cu_k[b + 1] - k0;
  if (kb * BN >= lk) return;
  const int grp = a.q_grp;
  const int hpp = a.k_hpp;                // query heads of this part
  const int h0 = g * grp + part * hpp;  // its first query head
  const bool causal = a.causal != 0;
  const SeqGeom sg{lq, lk, a.window, causal};
  TileRange qr = key_tile_queries(sg, kb, BN, BM);
  // with the mask's ranges: only query tiles in which some row has an allowed
  // bit for a key of this tile
  if constexpr (M)
    if (a.mask_ranges != nullptr) narrow_by_mask(a, false, b, kb * BN / 32, BN / 32, BM / 32, qr.lo, qr.hi);

  const int64_t qstride = (int64_t)a.heads_q * D;
  const int64_t kstride = (int64_t)a.heads_kv * D;
  const int j = kb * BN + 32 * kt + l32;  // this lane's key (rows past L_k hold copies; not stored)
  const bool key_ok = j < lk;
  {
    const int kvalid = min(BN, lk - kb * BN);
    const int64_t koff = (int64_t)(k0 + kb * BN) * kstride + g * D;
    const uint32_t sb = (uint32_t)(kstride * sizeof(T));
    TileLoader<T, BN, D, NT> kvld;
    kvld.init(sb, w, lane);
    kvld.issue(klds, static_cast<const T*>(a.k) + koff, sb, kvalid);
    kvld.issue(vlds, static_cast<const T*>(a.v) + koff, sb, kvalid);
  }
  RowReader<T, D> rrd;
  rrd.init(l32, half);
  ColReader<T, D> crd;
  crd.init(lane);
  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dka[dt] = f32x16{};
    dva[dt] = f32x16{};
  }
  const float c = a.scale * kLog2e;
  const PairWindow pw = pair_window(lq, lk, a.window, causal);
  const T* __restrict__ Qg = static_cast<const T*>(a.q);
  const T* __restrict__ Dg = static_cast<const T*>(a.dout);

  // Steps walk (head, query tile) pairs: head h0 .. h0+hpp-1 outer, query
  // tile qr.lo .. qr.hi inner. An empty range (no query sees this key tile)
  // has no steps and writes zeros.
  const int nq = qr.hi >= qr.lo ? qr.hi - qr.lo + 1 : 0;
  const int steps = hpp * nq;
  const uint32_t qsb = (uint32_t)(qstride * sizeof(T));
  TileLoader<T, BM, D, NT> qld;
  qld.init(qsb, w, lane);
  // Fill state, kept as running offsets so that a step costs a few scalar
  // adds: the next (head, query tile)'s element offset into Q and dO, its
  // index into the [Hq, T_q] LSE*log2e and D arrays and (with M) its word
  // offset into the mask. A fill advances one tile; after the range's last
  // tile it returns to the first tile of the next head (the mask is shared by
  // the heads, so its offset returns to the first tile's). Only the range's
  // last tile can be partial: its rows past L_q arrive as zeros (LSE*log2e
  // and D too) and are masked.
  const int64_t tile_elems = (int64_t)BM * qstride;
  int64_t qoff = (int64_t)(q0 + qr.lo * BM) * qstride + (int64_t)h0 * D;
  int64_t soff = (int64_t)h0 * a.total_q + q0 + qr.lo * BM;
  int64_t moff = (int64_t)(q0 + qr.lo * BM) * a.mask_words + 4 * kb;
  const int64_t qwrap = D - (int64_t)(nq - 1) * tile_elems;
  const int64_t swrap = (int64_t)a.total_q - (int64_t)(nq - 1) * BM;
  const int64_t mstep = (int64_t)BM * a.mask_words;
  const uint32_t last_rows = (uint32_t)min(BM, lq - qr.hi * BM);
  int nqb = qr.lo;  // query tile of the next step to fill
  auto fill = [&](char* st) {
    const bool last = nqb == qr.hi;
    const uint32_t qvalid = last ? last_rows : (uint32_t)BM;
    qld.issue(st, Qg + qoff, qsb, qvalid);
    qld.issue(st + QTile::kBytes, Dg + qoff, qsb, qvalid);
    if (w == 0) {
      buffer_to_lds4(buffer_rsrc(a.lse2 + soff, qvalid * 4u), st + 2 * QTile::kBytes, (uint32_t)lane * 4u);
      buffer_to_lds4(buffer_rsrc(a.delta + soff, qvalid * 4u), st + 2 * QTile::kBytes + BM * 4,
                     (uint32_t)lane * 4u);
    }
    if constexpr (M) {
      if (w == 1) {  // lane r: row r's words 4 kb .. 4 kb + 3; rows past L_q arrive as zeros
        const uint32_t rb = (uint32_t)a.mask_words * 4u;
        buffer_to_lds16(buffer_rsrc(a.mask + moff, qvalid * rb), st + kMaskOff, (uint32_t)lane * rb);
      }
    }
    if (last) {
      nqb = qr.lo;
      qoff += qwrap;
      soff += swrap;
      moff -= (int64_t)(nq - 1) * mstep;
    } else {
      ++nqb;
      qoff += tile_elems;
      soff += BM;
      moff += mstep;
    }
  };
  // odd step counts start in stage 1: the loop below runs whole stage pairs
  if (steps > 0) fill(steps & 1 ? st1 : st0);
  __syncthreads();

  // The query tiles whose tile with this key tile has every cell visible (no
  // per-cell mask), and those in which this wave's 32 keys x 32 queries see
  // at least one cell: intervals computed once, tested per step.
  const QbRange full_q = key_tile_full_query_tiles(sg, kb, BN, BM);
  const QbRange seen_q = block_seen_query_tiles(sg, BM, 32 * mh, 32, kb * BN + 32 * kt, 32);
  int qb = qr.lo;  // query tile of the current step
  auto step = [&](auto stage_c, int t) {
    constexpr int stage = decltype(stage_c)::value;
    const char* qs = stage ? st1 : st0;
    const char* dos = qs + QTile::kBytes;
    const float* lse2s = reinterpret_cast<const float*>(qs + 2 * QTile::kBytes);
    const float* dlts = lse2s + BM;
    const bool edge = qb < full_q.lo || qb > full_q.hi;
    // this wave's 32 keys x 32 queries all masked: P = dS = 0, nothing to add;
    // the wave skips both contraction phases but still fills and meets the
    // barrier
    const bool work = !edge || (seen_q.lo <= qb && qb <= seen_q.hi);
    f32x16 s, dp;  // set and read only when `work`
    f32x4 lsv[4];  // LSE * log2(e) of this lane's 16 query rows
    if (work) {
    s = f32x16{};
    // dP - D: the dP accumulator starts at -D of its rows (the workspace holds
    // -D), so dS = P * dP needs no subtraction per cell
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(dlts + 32 * mh + 8 * r4 + 4 * half);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[4 * r4 + e] = d4[e];
    }
#pragma unroll
    for (int ss = 0; ss < D / 16; ++ss) {
      mma(s, rrd.read(qs, 32 * mh, ss), rrd.read(klds, 32 * kt, ss));
      mma(dp, rrd.read(dos, 32 * mh, ss), rrd.read(vlds, 32 * kt, ss));
    }
    if (edge) {
      // row r holds query ib + 8(r/4) + r%4: visible iff it is a real row
      // (< L_q) and inside the window (pair_window) at p = query + L_k - L_q
      const int ib = qb * BM + 32 * mh + 4 * half;
      apply_visible(s, key_rows_visible(ib, ib + (lk - lq) - j + pw.off, lq, pw));
    }
    if constexpr (M) {  // this lane's key is bit l32 of word kt of each row
      const char* mt = qs + kMaskOff;
      uint32_t words[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        words[r] = *reinterpret_cast<const uint32_t*>(mt + 16 * (32 * mh + 4 * half + 8 * (r >> 2) + (r & 3)) + 4 * kt);
      apply_col_mask(s, words, l32);
    }
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) lsv[r4] = *reinterpret_cast<const f32x4*>(lse2s + 32 * mh + 8 * r4 + 4 * half);
    // P and dS = P (dP - D) of the first 16 query rows (registers 0..7) now;
    // the other 16 are formed between the first half's dV / dK MFMAs below
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float pv = fast_exp2(fmaf(s[r], c, -lsv[r >> 2][r & 3]));
      s[r] = pv;
      dp[r] = pv * dp[r];
    }
    }
    // the next step's stage is filled here, after this step's row reads and
    // softmax, not at the top of the step, where the loads met the burst of
    // row reads every wave makes (moving them here cut dK/dV time by 4%)
    if (t + 1 < steps) fill(stage ? st0 : st1);
    if (work) {
      // The two waves sharing a SIMD (the two query halves of one key block)
      // run the same phases at the same time, so a softmax that follows all
      // of the S / dP MFMAs finds the matrix core idle. Here each MFMA pair of
      // the first 16 rows is followed by the exp2, FMA and multiply of two
      // cells of the last 16 (four at head_dim 64), in one wave's instruction
      // stream, so that they issue while the matrix core works (scheduling
      // fences keep the order; each chunk reads the next chunk's operands
      // first). dK/dV 3.3-4.5% faster in four interleaved A/B runs, outputs
      // bitwise equal.
      const Frag<T> pf0 = acc_frag<T>(s, 0);
      const Frag<T> dsf0 = acc_frag<T>(dp, 0);
      Frag<T> a0 = crd.read(dos, 32 * mh, 0), b0 = crd.read(qs, 32 * mh, 0);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        // the next chunk's operands; after the last, the second half's first
        const int row1 = dt + 1 < D / 32 ? 32 * mh : 32 * mh + 16;
        const int dt1 = dt + 1 < D / 32 ? dt + 1 : 0;
        const Frag<T> a1 = crd.read(dos, row1, dt1), b1 = crd.read(qs, row1, dt1);
        mma(dva[dt], a0, pf0);
        mma(dka[dt], b0, dsf0);
#pragma unroll
        for (int e2 = 0; e2 < 8 / (D / 32); ++e2) {
          const int r = 8 + (8 / (D / 32)) * dt + e2;
          const float pv = fast_exp2(fmaf(s[r], c, -lsv[r >> 2][r & 3]));
          s[r] = pv;
          dp[r] = pv * dp[r];
        }
        __builtin_amdgcn_sched_barrier(0);
        a0 = a1;
        b0 = b1;
      }
      const Frag<T> pf1 = acc_frag<T>(s, 1);
      const Frag<T> dsf1 = acc_frag<T>(dp, 1);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        mma(dva[dt], dt == 0 ? a0 : crd.read(dos, 32 * mh + 16, dt), pf1);
        mma(dka[dt], dt == 0 ? b0 : crd.read(qs, 32 * mh + 16, dt), dsf1);
      }
    }
    if (++qb > qr.hi) qb = qr.lo;
    __syncthreads();
  };
  int t = 0;
  if (steps & 1) step(ic<1>{}, t++);
  for (; t < steps; t += 2) {
    step(ic<0>{}, t);
    step(ic<1>{}, t + 1);
  }

  // Sum the two query halves: half 1 hands its dK partial to half 0 and half 0
  // hands its dV partial to half 1, through fp32 LDS in the accumulator layout
  // (one 32-key block per wave, reusing the K/V tiles and the stages).
  float* red_k = reinterpret_cast<float*>((kt < 2 ? klds : vlds) + (kt & 1) * kRedBlock);
  float* red_v = reinterpret_cast<float*>((kt < 2 ? st0 : st1) + (kt & 1) * kRedBlock);
  // mh is wave-uniform: one branch around each whole loop (a branch per
  // element would make the compiler copy the accumulators at every one)
  if (steps > 0) {
    if (mh == 1) hand_over(red_k, dka, lane);
    else hand_over(red_v, dva, lane);
  }
  __syncthreads();
  if (steps > 0) {
    if (mh == 0) take_over(red_k, dka, lane);
    else take_over(red_v, dva, lane);
  }
  if (key_ok) {
    const int64_t roff = (int64_t)(k0 + j) * kstride + g * D;
    if (a.kv_split == 1) {
      if (mh == 0) store_acc_rows<T, D>(static_cast<T*>(a.dk) + roff, dka, a.scale, half);
      else store_acc_rows<T, D>(static_cast<T*>(a.dv) + roff, dva, 1.f, half);
    } else {  // this part's fp32 partial sums; bwd_dkdv_sum_kernel adds the parts
      float* pk = a.dkv_part + (int64_t)part * 2 * a.total_k * kstride;
      if (mh == 0) store_acc_rows<float, D>(pk + roff, dka, 1.f, half);
      else store_acc_rows<float, D>(pk + (int64_t)a.total_k * kstride + roff, dva, 1.f, half);
    }
  }
}

// dK = scale * (sum of the parts' dK partials) and dV = sum of the dV
// partials, converted to T: 4 consecutive elements per thread. Every key row
// of every sequence was written by every part (zeros where no query sees it).
template <typename T>
__global__ void __launch_bounds__(256) bwd_dkdv_sum_kernel(AttnArgs a, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const int64_t n = n4 * 4;  // elements of dK (and of dV)
  f32x4 k4 = {0.f, 0.f, 0.f, 0.f}, v4 = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < a.kv_split; ++p) {
    const float* pk = a.dkv_part + (int64_t)p * 2 * n;
    k4 += *reinterpret_cast<const f32x4*>(pk + 4 * i);
    v4 += *reinterpret_cast<const f32x4*>(pk + n + 4 * i);
  }
  store4<T>(static_cast<T*>(a.dk) + 4 * i, k4[0] * a.scale, k4[1] * a.scale, k4[2] * a.scale, k4[3] * a.scale);
  store4<T>(static_cast<T*>(a.dv) + 4 * i, v4[0], v4[1], v4[2], v4[3]);
}

// ------------------------------------------ backward: dK, dV at head_dim 256
// One workgroup per (KV head, sequence, key tile of BN = 128 keys), 4 waves, one
// per SIMD: wave w owns keys 32*w .. +31 and all 256 head dims of their dK and
// dV, with its keys' K and V rows in registers (64 + 64). The (head, query
// tile) steps run twice: the first pass forms S and P and accumulates dV, the
// second forms S, dP and dS and accumulates dK, so only one 128-register
// accumulator is live at a time (dK and dV together, with S and dP, would not
// fit the accumulator registers). LDS holds only the two stages of the
// streamed query tiles (Q, dO, LSE*log2e, D), BM = 32 queries per step.
template <typename T, int D, int BN, int BM, bool M>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_dkdv_wide_kernel(AttnArgs a) {
  constexpr int NT = 256;
  static_assert((D == 256 || D == 512) && BN == 128 && BM == 32,
                "wave layout assumes 4 key blocks of 32 keys, all dims per wave");
  // accumulator columns per pass: all 256 at head_dim 256; at 512 the dV and
  // dK passes each run four times, over columns 0-127, ..., 384-511
  constexpr int DA = D > 256 ? 128 : D;
  constexpr int NH = D / DA;
  using QTile = LdsTile<T, BM, D>;
  constexpr int kStats = 64 * 4;  // one 64-lane 4-byte load's worth
  // with M, the step's mask tile follows: one 16-byte load per lane (rows past
  // BM arrive as zeros), the 4 words of this key tile's 128 keys per row
  constexpr int kMaskOff = 2 * QTile::kBytes + 2 * kStats;
  constexpr int kStage = kMaskOff + (M ? 64 * 16 : 0);  // Q, dO, LSE*log2e, D[, mask]
  __shared__ __attribute__((aligned(1024))) char st0[kStage];
  __shared__ __attribute__((aligned(1024))) char st1[kStage];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int w = wave_uniform(tid >> 6);
  static_assert(BN == 128, "the launch-id decode counts 128-key tiles (AttnArgs::k_nkb)");
  const int nkb = a.k_nkb;
  uint32_t L = (uint32_t)xcd_remap((int)blockIdx.x, a.k_items);  // kv_split is 1 here
  uint32_t qt = fast_div(L, a.div_nkb);
  const int kb = (int)(L - qt * (uint32_t)nkb);
  L = qt;
  qt = fast_div(L, a.div_batch);
  const int b = (int)(L - qt * (uint32_t)a.batch);
  const int g = (int)qt;
  const int q0 = a.cu_q[b], lq = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], lk = a.cu_k[b + 1] - k0;
  if (kb * BN >= lk) return;
  const int grp = a.q_grp;
  const bool causal = a.causal != 0;
  const SeqGeom sg{lq, lk, a.window, causal};
  TileRange qr = key_tile_queries(sg, kb, BN, BM);
  // with the mask's ranges: only query tiles in which some row has an allowed
  // bit for a key of this tile
  if constexpr (M)
    if (a.mask_ranges != nullptr) narrow_by_mask(a, false, b, kb * BN / 32, BN / 32, BM / 32, qr.lo, qr.hi);

  const int64_t qstride = (int64_t)a.heads_q * D;
  const int64_t kstride = (int64_t)a.heads_kv * D;
  const int j = kb * BN + 32 * w + l32;  // this lane's key (rows past L_k are zeros; not stored)
  const bool key_ok = j < lk;
  Frag<T> kf[D / 16], vf[D / 16];
  {
    const int64_t roff = (int64_t)(k0 + (key_ok ? j : 0)) * kstride + g * D + 8 * half;
    const T* krow = static_cast<const T*>(a.k) + roff;
    const T* vrow = static_cast<const T*>(a.v) + roff;
#pragma unroll
    for (int ss = 0; ss < D / 16; ++ss) {
      kf[ss] = key_ok ? global_frag<T>(krow + 16 * ss) : zero_frag<T>();
      vf[ss] = key_ok ? global_frag<T>(vrow + 16 * ss) : zero_frag<T>();
    }
  }
  RowReader<T, D> rrd;
  rrd.init(l32, half);
  ColReader<T, D> crd;
  crd.init(lane);
  const float c = a.scale * kLog2e;
  const PairWindow pw = pair_window(lq, lk, a.window, causal);
  const T* __restrict__ Qg = static_cast<const T*>(a.q);
  const T* __restrict__ Dg = static_cast<const T*>(a.dout);

  // (head, query tile) steps as in the 128-key kernel, walked once per pass;
  // an empty range writes zeros
  const int nq = qr.hi >= qr.lo ? qr.hi - qr.lo + 1 : 0;
  const int steps = grp * nq;
  int nh = g * grp, nqb = qr.lo;  // (head, query tile) of the next step to fill
  const uint32_t qsb = (uint32_t)(qstride * sizeof(T));
  TileLoader<T, BM, D, NT> qld;
  qld.init(qsb, w, lane);
  auto fill = [&](char* st) {
    const int qvalid = min(BM, lq - nqb * BM);
    const int64_t qoff = (int64_t)(q0 + nqb * BM) * qstride + nh * D;
    qld.issue(st, Qg + qoff, qsb, qvalid);
    qld.issue(st + QTile::kBytes, Dg + qoff, qsb, qvalid);
    if (w == 0) {  // 64 lanes, BM = 32 rows: lanes past qvalid read zeros
      const int64_t idx = (int64_t)nh * a.total_q + q0 + nqb * BM;
      buffer_to_lds4(buffer_rsrc(a.lse2 + idx, (uint32_t)qvalid * 4u), st + 2 * QTile::kBytes, (uint32_t)lane * 4u);
      buffer_to_lds4(buffer_rsrc(a.delta + idx, (uint32_t)qvalid * 4u), st + 2 * QTile::kBytes + kStats,
                     (uint32_t)lane * 4u);
    }
    if constexpr (M) {
      if (w == 1) {  // lane r: row r's words 4 kb .. 4 kb + 3; rows past L_q arrive as zeros
        const uint32_t rb = (uint32_t)a.mask_words * 4u;
        buffer_to_lds16(buffer_rsrc(a.mask + (int64_t)(q0 + nqb * BM) * a.mask_words + 4 * kb, (uint32_t)qvalid * rb),
                        st + kMaskOff, (uint32_t)lane * rb);
      }
    }
    if (++nqb > qr.hi) {
      nqb = qr.lo;
      if (++nh == g * grp + grp) nh = g * grp;  // the next pass starts over
    }
  };
  const int total = 2 * NH * steps;
  // odd step counts start in stage 1: the loops below run whole stage pairs
  if (total > 0) fill(steps & 1 ? st1 : st0);
  __syncthreads();

  int qb = qr.lo;  // query tile of the current step
  // S for this wave's 32 keys against the stage's 32 query rows, masked, and
  // the rows' LSE * log2(e); returns false when the whole block is masked.
  // The exp2 that turns S into P is left to the passes: with one wave per
  // SIMD nothing else hides the softmax, so each pass issues it between its
  // own MFMAs (the dV pass between the MFMAs of the first 16 rows, the dK
  // pass beside the dP MFMAs, which do not need P), ordered by scheduling
  // fences, with the next operand read issued first.
  auto scores = [&](const char* qs, f32x16& s, f32x4 (&lsv)[4]) -> bool {
    const bool edge = !tile_full_i32(lq, lk, a.window, causal, qb, BM, kb, BN);
    if (edge && block_masked(lq, lk, a.window, causal, qb * BM, BM, kb * BN + 32 * w, 32)) return false;
    s = f32x16{};
#pragma unroll
    for (int ss = 0; ss < D / 16; ++ss) mma(s, rrd.read(qs, 0, ss), kf[ss]);
    if (edge) {
      const int ib = qb * BM + 4 * half;
      apply_visible(s, key_rows_visible(ib, ib + (lk - lq) - j + pw.off, lq, pw));
    }
    if constexpr (M) {  // this lane's key is bit l32 of word w of each row
      const char* mt = qs + kMaskOff;
      uint32_t words[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        words[r] = *reinterpret_cast<const uint32_t*>(mt + 16 * (4 * half + 8 * (r >> 2) + (r & 3)) + 4 * w);
      apply_col_mask(s, words, l32);
    }
    const float* lse2s = reinterpret_cast<const float*>(qs + 2 * QTile::kBytes);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) lsv[r4] = *reinterpret_cast<const f32x4*>(lse2s + 8 * r4 + 4 * half);
    return true;
  };
  auto next = [&]() {  // end of a step: advance the query tile, meet the stage barrier
    if (++qb > qr.hi) qb = qr.lo;
    __syncthreads();
  };

  // Steps t0 .. t0 + steps - 1 of one pass: global step t runs on stage
  // (t + steps % 2) % 2 (the first fill went to stage steps % 2), so a pass
  // may start with a lone stage-1 step and end with a lone stage-0 step, with
  // whole stage pairs between
  auto run = [&](auto step, int t0) __attribute__((always_inline)) {
    int t = t0;
    const int end = t0 + steps;
    if (t < end && ((t + (steps & 1)) & 1)) step(ic<1>{}, t++);
    for (; t + 1 < end; t += 2) {
      step(ic<0>{}, t);
      step(ic<1>{}, t + 1);
    }
    if (t < end) step(ic<0>{}, t);
  };

  // dV passes: dV += P^T dO, columns DA h .. DA h + DA - 1
  auto dv_pass = [&](auto h_c) __attribute__((always_inline)) {
    constexpr int h = decltype(h_c)::value;
    f32x16 dva[DA / 32];
#pragma unroll
    for (int dt = 0; dt < DA / 32; ++dt) dva[dt] = f32x16{};
    auto step = [&](auto stage_c, int t) {
      constexpr int stage = decltype(stage_c)::value;
      const char* qs = stage ? st1 : st0;
      const char* dos = qs + QTile::kBytes;
      if (t + 1 < total) fill(stage ? st0 : st1);
      f32x16 s;
      f32x4 lsv[4];
      if (scores(qs, s, lsv)) {
        // P of the first 16 rows; the last 16 rows' exp2 issue between the
        // first half's MFMAs (a cell per chunk at 256 output columns, two
        // at 128)
#pragma unroll
        for (int r = 0; r < 8; ++r) s[r] = fast_exp2(fmaf(s[r], c, -lsv[r >> 2][r & 3]));
        const Frag<T> pf0 = acc_frag<T>(s, 0);
        Frag<T> a0 = crd.read(dos, 0, h * (DA / 32));
#pragma unroll
        for (int dt = 0; dt < DA / 32; ++dt) {
          const Frag<T> a1 = crd.read(dos, dt + 1 < DA / 32 ? 0 : 16, h * (DA / 32) + (dt + 1) % (DA / 32));
          mma(dva[dt], a0, pf0);
#pragma unroll
          for (int r = 8; r < 16; ++r)
            if ((r - 8) * (DA / 32) / 8 == dt) s[r] = fast_exp2(fmaf(s[r], c, -lsv[r >> 2][r & 3]));
          __builtin_amdgcn_sched_barrier(0);
          a0 = a1;
        }
        const Frag<T> pf1 = acc_frag<T>(s, 1);
#pragma unroll
        for (int dt = 0; dt < DA / 32; ++dt) mma(dva[dt], dt == 0 ? a0 : crd.read(dos, 16, h * (DA / 32) + dt), pf1);
      }
      next();
    };
    run(step, h * steps);
    if (key_ok)
      store_acc_rows<T, DA>(static_cast<T*>(a.dv) + (int64_t)(k0 + j) * kstride + g * D + h * DA, dva, 1.f, half);
  };
  // dK passes: dK += dS^T Q with dS = P (dP - D), columns DA h .. DA h + DA - 1
  auto dk_pass = [&](auto h_c) __attribute__((always_inline)) {
    constexpr int h = decltype(h_c)::value;
    f32x16 dka[DA / 32];
#pragma unroll
    for (int dt = 0; dt < DA / 32; ++dt) dka[dt] = f32x16{};
    auto step = [&](auto stage_c, int t) {
      constexpr int stage = decltype(stage_c)::value;
      const char* qs = stage ? st1 : st0;
      const char* dos = qs + QTile::kBytes;
      const float* dlts = reinterpret_cast<const float*>(qs + 2 * QTile::kBytes + kStats);
      if (t + 1 < total) fill(stage ? st0 : st1);
      f32x16 s;
      f32x4 lsv[4];
      if (scores(qs, s, lsv)) {
        // dP's MFMAs do not need P: its exp2 issue between them, a cell per
        // MFMA at head_dim 256, one every other MFMA at 512
        f32x16 dp = f32x16{};
        {
          Frag<T> b0 = rrd.read(dos, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ss = 0; ss < D / 16; ++ss) {
            const Frag<T> b1 = rrd.read(dos, 0, (ss + 1) % (D / 16));
            mma(dp, b0, vf[ss]);
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (r * (D / 16) / 16 == ss) s[r] = fast_exp2(fmaf(s[r], c, -lsv[r >> 2][r & 3]));
            __builtin_amdgcn_sched_barrier(0);
            b0 = b1;
          }
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dlts + 8 * r4 + 4 * half);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[4 * r4 + e] = s[4 * r4 + e] * (dp[4 * r4 + e] + d4[e]);  // dS (d4: -D)
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const Frag<T> dsf = acc_frag<T>(dp, u);
#pragma unroll
          for (int dt = 0; dt < DA / 32; ++dt) mma(dka[dt], crd.read(qs, 16 * u, h * (DA / 32) + dt), dsf);
        }
      }
      next();
    };
    run(step, (NH + h) * steps);
    if (key_ok)
      store_acc_rows<T, DA>(static_cast<T*>(a.dk) + (int64_t)(k0 + j) * kstride + g * D + h * DA, dka, a.scale,
                            half);
  };
  dv_pass(ic<0>{});
  if constexpr (NH > 1) dv_pass(ic<1>{});
  if constexpr (NH > 2) {
    dv_pass(ic<2>{});
    dv_pass(ic<3>{});
  }
  dk_pass(ic<0>{});
  if constexpr (NH > 1) dk_pass(ic<1>{});
  if constexpr (NH > 2) {
    dk_pass(ic<2>{});
    dk_pass(ic<3>{});
  }
}

// ------------------------------------------------ backward: dK, dV (4 waves)
// The general dK/dV kernel (used for fp32, whose tiles are twice as large):
// 4 waves of 32 keys, K and V in registers, 64-query steps.
// Key-major decode: KV head outermost, then sequence, then key tile ascending
// (for the causal mask early key tiles are seen by the most queries).
template <typename T, int D, int BN, int BM, bool M>
__global__ void __launch_bounds__(BN * 2) bwd_dkdv4_kernel(AttnArgs a) {
  constexpr int NT = BN * 2;
  using QTile = LdsTile<T, BM, D>;
  // with M, the step's mask tile follows: BM rows x 4 words (this key tile's
  // 128 keys)
  static_assert(BM == 64, "one 64-lane load per row for LSE*log2e, D and the mask");
  constexpr int kMaskOff = 2 * QTile::kBytes + 2 * BM * 4;
  constexpr int kStage = kMaskOff + (M ? BM * 16 : 0);  // Q, dO, LSE*log2e, D[, mask]
  __shared__ __attribute__((aligned(1024))) char st0[kStage];
  __shared__ __attribute__((aligned(1024))) char st1[kStage];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  static_assert(BN == 128, "the launch-id decode counts 128-key tiles (AttnArgs::k_nkb)");
  const int nkb = a.k_nkb;
  uint32_t L = (uint32_t)xcd_remap((int)blockIdx.x, a.k_items);  // kv_split is 1 here
  uint32_t qt = fast_div(L, a.div_nkb);
  const int kb = (int)(L - qt * (uint32_t)nkb);
  L = qt;
  qt = fast_div(L, a.div_batch);
  const int b = (int)(L - qt * (uint32_t)a.batch);
  const int g = (int)qt;
  const int q0 = a.cu_q[b], lq = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], lk = a.cu_k[b + 1] - k0;
  if (kb * BN >= lk) return;
  const int grp = a.q_grp;
  const SeqGeom sg{lq, lk, a.window, a.causal != 0};
  TileRange qr = key_tile_queries(sg, kb, BN, BM);
  // with the mask's ranges: only query tiles in which some row has an allowed
  // bit for a key of this tile
  if constexpr (M)
    if (a.mask_ranges != nullptr) narrow_by_mask(a, false, b, kb * BN / 32, BN / 32, BM / 32, qr.lo, qr.hi);

  const int64_t qstride = (int64_t)a.heads_q * D;
  const int64_t kstride = (int64_t)a.heads_kv * D;
  const int j = kb * BN + w * 32 + l32;  // this lane's key
  const bool key_ok = j < lk;
  Frag<T> kf[D / 16], vf[D / 16];
  {
    const int64_t roff = (int64_t)(k0 + (key_ok ? j : 0)) * kstride + g * D + 8 * half;
    const T* krow = static_cast<const T*>(a.k) + roff;
    const T* vrow = static_cast<const T*>(a.v) + roff;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      kf[s] = key_ok ? global_frag<T>(krow + 16 * s) : zero_frag<T>();
      vf[s] = key_ok ? global_frag<T>(vrow + 16 * s) : zero_frag<T>();
    }
  }
  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dka[dt] = f32x16{};
    dva[dt] = f32x16{};
  }
  const float c = a.scale * kLog2e;
  const bool causal = a.causal != 0;
  const PairWindow pw = pair_window(lq, lk, a.window, causal);
  const T* __restrict__ Qg = static_cast<const T*>(a.q);
  const T* __restrict__ Dg = static_cast<const T*>(a.dout);

  // Steps t = 0 .. grp * nq - 1 walk (head, query tile) pairs; an empty range
  // (no query sees this key tile) has no steps and writes zeros.
  const int nq = qr.hi >= qr.lo ? qr.hi - qr.lo + 1 : 0;
  const int steps = grp * nq;
  // The streamed tiles go from HBM straight into LDS (no staging registers:
  // with K and V rows and both accumulators in registers, a register-staged
  // copy made this kernel spill). Rows past L_q arrive as zeros (LSE*log2e
  // and D too) and are masked.
  const uint32_t qsb = (uint32_t)(qstride * sizeof(T));
  TileLoader<T, BM, D, NT> qld;
  qld.init(qsb, w, lane);
  auto fill = [&](int t, char* st) {
    const int h = g * grp + t / nq;
    const int qb = qr.lo + t % nq;
    const uint32_t qvalid = (uint32_t)min(BM, lq - qb * BM);
    const int64_t qoff = (int64_t)(q0 + qb * BM) * qstride + h * D;
    qld.issue(st, Qg + qoff, qsb, qvalid);
    qld.issue(st + QTile::kBytes, Dg + qoff, qsb, qvalid);
    if (w == 0) {
      const int64_t idx = (int64_t)h * a.total_q + q0 + qb * BM;
      buffer_to_lds4(buffer_rsrc(a.lse2 + idx, qvalid * 4u), st + 2 * QTile::kBytes, (uint32_t)lane * 4u);
      buffer_to_lds4(buffer_rsrc(a.delta + idx, qvalid * 4u), st + 2 * QTile::kBytes + BM * 4,
                     (uint32_t)lane * 4u);
    }
    if constexpr (M) {
      if (w == 1) {  // lane r: row r's words 4 kb .. 4 kb + 3
        const uint32_t rb = (uint32_t)a.mask_words * 4u;
        buffer_to_lds16(buffer_rsrc(a.mask + (int64_t)(q0 + qb * BM) * a.mask_words + 4 * kb, qvalid * rb),
                        st + kMaskOff, (uint32_t)lane * rb);
      }
    }
  };
  if (steps > 0) fill(0, st0);
  __syncthreads();

  for (int t = 0; t < steps; ++t) {
    const int stage = t & 1;
    const char* qs = stage ? st1 : st0;
    const char* dos = qs + QTile::kBytes;
    const float* lse2s = reinterpret_cast<const float*>(qs + 2 * QTile::kBytes);
    const float* dlts = lse2s + BM;
    const int qb = qr.lo + t % nq;
    if (t + 1 < steps) fill(t + 1, stage ? st0 : st1);
    const bool edge = pw.windowed && !tile_is_full(sg, qb, BM, kb, BN);
    // one 32-row block at a time (unrolled, the two blocks' fragments were
    // live together and spilled)
#pragma unroll 1
    for (int mt = 0; mt < BM / 32; ++mt) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ss = 0; ss < D / 16; ++ss) {
        mma(s, row_frag<T, BM, D>(qs, 32 * mt + l32, 2 * ss + half), kf[ss]);
        mma(dp, row_frag<T, BM, D>(dos, 32 * mt + l32, 2 * ss + half), vf[ss]);
      }
      if (edge) {
        // row r holds query qb*BM + 32mt + 8(r/4) + 4half + r%4; visible iff
        // inside the window (pair_window) at p = query + L_k - L_q
        const int mb = qb * BM + 32 * mt + 4 * half + (lk - lq) - j + pw.off;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((uint32_t)(mb + 8 * (r >> 2) + (r & 3)) >= pw.lim) s[r] = -INFINITY;
      }
      if constexpr (M) {  // this lane's key is bit l32 of word w of each row
        const uint32_t* mt4 = reinterpret_cast<const uint32_t*>(qs + kMaskOff);
        uint32_t words[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) words[r] = mt4[4 * (32 * mt + 4 * half + 8 * (r >> 2) + (r & 3)) + w];
        apply_col_mask(s, words, l32);
      }
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int rr = 32 * mt + 8 * r4 + 4 * half;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + rr);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dlts + rr);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          const float pv = fast_exp2(fmaf(s[r], c, -l4[e]));
          s[r] = pv;
          dp[r] = pv * (dp[r] + d4[e]);  // dS (d4: -D)
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const Frag<T> pf = acc_frag<T>(s, u);
        const Frag<T> dsf = acc_frag<T>(dp, u);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          mma(dva[dt], col_frag<T, BM, D>(dos, 32 * mt + 16 * u, 32 * dt, lane), pf);
          mma(dka[dt], col_frag<T, BM, D>(qs, 32 * mt + 16 * u, 32 * dt, lane), dsf);
        }
      }
    }
    __syncthreads();
  }
  if (key_ok) {
    const int64_t roff = (int64_t)(k0 + j) * kstride + g * D;
    store_acc_rows<T, D>(static_cast<T*>(a.dk) + roff, dka, a.scale, half);
    store_acc_rows<T, D>(static_cast<T*>(a.dv) + roff, dva, 1.f, half);
  }
}

// ---------------------------------------------------------------- launchers
// Tile shapes (every dtype): forward and dQ take 4 waves of 32 query rows (4,
// 2 or 1 heads of a KV group x 32, 64 or 128 rows; query_heads_per_wg) and
// step over keys 64 at a time. dK/dV takes 128 keys (8 waves: 4 key
// blocks of 32 x 2 query halves; fp32: 4 waves) and steps over queries 64 at a
// time; at head_dim 256 it takes 128 keys (4 waves of 32 keys, two passes) and
// steps over queries 32 at a time.
template <int D> struct Tiles {
  static constexpr int kFwdBM = 128, kFwdBN = D > 256 ? 32 : 64;
  static constexpr int kBwdBN = 128, kBwdBM = D > 128 ? 32 : 64;
};

// The launch-invariant parts of the launch-id decode (AttnArgs::q_*, k_*,
// div_*), for query-major tiles of 128 rows over 1, 2 or 4 heads and
// key-major tiles of 128 keys. The C ABI bounds both item counts by INT32_MAX.
static AttnArgs with_decode(const AttnArgs& in) {
  AttnArgs a = in;
  const int hw = query_heads_per_wg(a.heads_q, a.heads_kv);
  a.q_grp = a.heads_q / a.heads_kv;
  a.q_hw_log2 = hw == 4 ? 2 : (hw == 2 ? 1 : 0);
  a.q_nch = a.q_grp / hw;
  a.q_rows = 128 / hw;
  a.q_nqb = (int32_t)(((int64_t)a.max_seqlen_q + a.q_rows - 1) / a.q_rows);
  a.q_items = (int32_t)((int64_t)a.q_nqb * a.q_nch * a.heads_kv * a.batch);
  a.k_nkb = (int32_t)(((int64_t)a.max_seqlen_k + 127) / 128);
  a.k_hpp = a.q_grp / a.kv_split;
  a.k_items = (int32_t)((int64_t)a.k_nkb * a.heads_kv * a.batch * a.kv_split);
  a.div_nch = make_fast_div((uint32_t)a.q_nch);
  a.div_nqb = make_fast_div((uint32_t)(a.q_nqb > 0 ? a.q_nqb : 1));
  a.div_batch = make_fast_div((uint32_t)a.batch);
  a.div_nkb = make_fast_div((uint32_t)(a.k_nkb > 0 ? a.k_nkb : 1));
  a.div_split = make_fast_div((uint32_t)a.kv_split);
  return a;
}

// M: a mask combined with the window (a.mask != nullptr)
template <typename T, int D, bool M>
static hipError_t launch_fwd_m(const AttnArgs& a, hipStream_t st) {
  using TL = Tiles<D>;
  const int64_t grid = a.q_items;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_kernel<T, D, TL::kFwdBM, TL::kFwdBN, M>), dim3((unsigned)grid), dim3(TL::kFwdBM * 2), 0,
                     st, a);
  return hipGetLastError();
}
template <typename T, int D>
static hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t st) {
  return a.mask != nullptr ? launch_fwd_m<T, D, true>(a, st) : launch_fwd_m<T, D, false>(a, st);
}

template <typename T, int D, bool M>
static hipError_t launch_bwd_m(int stages, const AttnArgs& a, hipStream_t st) {
  using TL = Tiles<D>;
  const int64_t rows = (int64_t)a.total_q * a.heads_q;
  hipError_t e = hipSuccess;
  // dQ forms D and LSE*log2e for its rows itself, so the D preprocess runs
  // only when dQ is not part of the call
  if ((stages & 1) && !(stages & 2) && rows > 0) {
    const int64_t tpb = delta_tokens_per_block<D>();
    const int64_t g0 = (a.total_q + tpb - 1) / tpb * a.heads_q;
    hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3((unsigned)g0), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & 2) {
    const int64_t g1 = a.q_items;
    if (g1 > 0 && rows > 0) {
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, TL::kFwdBM, TL::kFwdBN, M>), dim3((unsigned)g1), dim3(TL::kFwdBM * 2),
                         0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  static_assert(TL::kBwdBN == 128, "with_decode counts 128-key tiles");
  const int64_t g2 = a.k_items;  // key tiles x KV heads x sequences x kv_split
  if ((stages & 4) && g2 > 0) {
    if constexpr (D > 128)
      hipLaunchKernelGGL((bwd_dkdv_wide_kernel<T, D, TL::kBwdBN, TL::kBwdBM, M>), dim3((unsigned)g2), dim3(256), 0,
                         st, a);
    else if constexpr (sizeof(T) == 2) {
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, TL::kBwdBN, TL::kBwdBM, M>), dim3((unsigned)g2),
                         dim3(TL::kBwdBN * 4), 0, st, a);
      if (a.kv_split > 1) {
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int64_t n4 = (int64_t)a.total_k * a.heads_kv * D / 4;
        if (n4 > 0)
          hipLaunchKernelGGL((bwd_dkdv_sum_kernel<T>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a, n4);
      }
    }
    else
      hipLaunchKernelGGL((bwd_dkdv4_kernel<T, D, TL::kBwdBN, TL::kBwdBM, M>), dim3((unsigned)g2),
                         dim3(TL::kBwdBN * 2), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}
template <typename T, int D>
static hipError_t launch_bwd_t(int stages, const AttnArgs& a, hipStream_t st) {
  return a.mask != nullptr ? launch_bwd_m<T, D, true>(stages, a, st) : launch_bwd_m<T, D, false>(stages, a, st);
}

// head_dim 256 and 512 exist for the 16-bit types only (the C ABI refuses
// fp32 there)
hipError_t launch_fwd(int dtype, int head_dim, const AttnArgs& in, hipStream_t st) {
  const AttnArgs a = with_decode(in);
  if (dtype == 2 && head_dim == 512) return launch_fwd_t<fp16, 512>(a, st);
  if (dtype == 1 && head_dim == 512) return launch_fwd_t<bf16, 512>(a, st);
  if (dtype == 2 && head_dim == 256) return launch_fwd_t<fp16, 256>(a, st);
  if (dtype == 2 && head_dim == 128) return launch_fwd_t<fp16, 128>(a, st);
  if (dtype == 2 && head_dim == 64) return launch_fwd_t<fp16, 64>(a, st);
  if (dtype == 1 && head_dim == 256) return launch_fwd_t<bf16, 256>(a, st);
  if (dtype == 1 && head_dim == 128) return launch_fwd_t<bf16, 128>(a, st);
  if (dtype == 1 && head_dim == 64) return launch_fwd_t<bf16, 64>(a, st);
  if (dtype == 0 && head_dim == 128) return launch_fwd_t<float, 128>(a, st);
  if (dtype == 0 && head_dim == 64) return launch_fwd_t<float, 64>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(int dtype, int head_dim, int stages, const AttnArgs& in, hipStream_t st) {
  const AttnArgs a = with_decode(in);
  if (dtype == 2 && head_dim == 512) return launch_bwd_t<fp16, 512>(stages, a, st);
  if (dtype == 1 && head_dim == 512) return launch_bwd_t<bf16, 512>(stages, a, st);
  if (dtype == 2 && head_dim == 256) return launch_bwd_t<fp16, 256>(stages, a, st);
  if (dtype == 2 && head_dim == 128) return launch_bwd_t<fp16, 128>(stages, a, st);
  if (dtype == 2 && head_dim == 64) return launch_bwd_t<fp16, 64>(stages, a, st);
  if (dtype == 1 && head_dim == 256) return launch_bwd_t<bf16, 256>(stages, a, st);
  if (dtype == 1 && head_dim == 128) return launch_bwd_t<bf16, 128>(stages, a, st);
  if (dtype == 1 && head_dim == 64) return launch_bwd_t<bf16, 64>(stages, a, st);
  if (dtype == 0 && head_dim == 128) return launch_bwd_t<float, 128>(stages, a, st);
  if (dtype == 0 && head_dim == 64) return launch_bwd_t<float, 64>(stages, a, st);
  return hipErrorInvalidValue;
}

// ------------------------------------------ scratch of the no-allocation backward
// D and LSE * log2(e) for callers that cannot allocate device memory: a fixed
// array in the code object, one copy per GPU, held until the process ends. On
// the host `scratch` names a host-side stand-in, never the device memory: its
// device address is looked up once per GPU, with that GPU current, and only
// that address reaches kernels.
static __device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(int device, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[device] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *ptr = addr[device];
  return hipSuccess;
}

template <int D> static void tiles_of(int* fwd_bm, int* fwd_bn, int* bwd_bn, int* bwd_bm) {
  *fwd_bm = Tiles<D>::kFwdBM;
  *fwd_bn = Tiles<D>::kFwdBN;
  *bwd_bn = Tiles<D>::kBwdBN;
  *bwd_bm = Tiles<D>::kBwdBM;
}

// Parts the dK/dV launch splits each KV group's query heads into: 1 when the
// key-major grid (key tiles x KV heads x sequences) already has a workgroup
// for each of the 256 compute units, else the fewest halvings of the group
// that reach that many (the 8-wave 16-bit kernel only).
int dkdv_split(int dtype, int head_dim, int heads_q, int heads_kv, int batch, int max_seqlen_k) {
  if (dtype == 0 || head_dim > 128) return 1;
  const int64_t g2 = (((int64_t)max_seqlen_k + Tiles<128>::kBwdBN - 1) / Tiles<128>::kBwdBN) * heads_kv * batch;
  const int grp = heads_q / heads_kv;
  int s = 1;
  while (g2 * s < 256 && grp % (2 * s) == 0) s *= 2;
  return s;
}

hipError_t launch_mask_ranges(const AttnArgs& a, int32_t* ranges, hipStream_t st) {
  const int nrb = (int)(((int64_t)a.max_seqlen_q + 31) / 32), nkb32 = (int)(((int64_t)a.max_seqlen_k + 31) / 32);
  const int64_t blocks = (int64_t)a.batch * (nrb + nkb32);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mask_range_kernel, dim3((unsigned)blocks), dim3(64), 0, st, a, ranges, nrb, nkb32);
  return hipGetLastError();
}

bool tile_sizes(int dtype, int head_dim, int* fwd_bm, int* fwd_bn, int* bwd_bn, int* bwd_bm) {
  if (dtype != 0 && dtype != 1 && dtype != 2) return false;
  if (head_dim == 64) tiles_of<64>(fwd_bm, fwd_bn, bwd_bn, bwd_bm);
  else if (head_dim == 128) tiles_of<128>(fwd_bm, fwd_bn, bwd_bn, bwd_bm);
  else if (head_dim == 256 && dtype != 0) tiles_of<256>(fwd_bm, fwd_bn, bwd_bn, bwd_bm);
  else if (head_dim == 512 && dtype != 0) tiles_of<512>(fwd_bm, fwd_bn, bwd_bn, bwd_bm);
  else return false;
  return true;
}

}  // namespace swa
