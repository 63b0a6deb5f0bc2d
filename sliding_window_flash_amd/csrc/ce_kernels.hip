// Linear cross-entropy without the logits tensor, for gfx950.
//
// The mlx-train-perf README's logit-free loss passage: the forward regenerates
// the logits z = H W^T tile by tile over the vocabulary and returns three
// per-token arrays (the loss, the log-sum-exp and the target logit); the
// backward recomputes the tiles it needs and returns the gradient into the
// hidden states only. Its backward walks the vocabulary in chunks, the one
// bounded intermediate being a chunk of dz = dL/dz.
//
//   forward  ce_logits_kernel<.., kFwd>: 256 vocab x 256 token tiles of
//            z^T = W H^T on MFMA (K = hidden size, 64 per step); each tile's
//            epilogue reduces its 256 logits per token to (max, sum of exp)
//            in the exp2 domain and picks the target logit when the target
//            falls in the tile. ce_reduce_kernel folds the per-tile partials
//            into LSE and the loss.
//   backward per vocabulary chunk [v0, v0 + vc):
//            ce_logits_kernel<.., kDz>: 256 token x 256 vocab tiles of
//            z = H W^T; dz = g (exp(z - LSE) - [v == y]) rounded to the I/O
//            type into the chunk buffer [n, vc];
//            ce_dh_kernel: dH += dz W_chunk, 256 token x 256 hidden tiles on
//            MFMA (K = the chunk's vocabulary, 64 per step), accumulated in
//            fp32 across chunks and written in the I/O type by the last.
#include <math.h>

#include "ce_launch.hpp"
#include "kernel_common.hpp"
#include "sched.hpp"

namespace swa {

namespace {

constexpr int kTile = 256;  // M and N tile rows
constexpr int kBK = 64;     // K per step
constexpr int kThreads = 512;
constexpr int kFwd = 0, kDz = 1;

// Workgroup -> (M tile, N tile): each XCD takes a contiguous run of ids; in
// that run, groups of kGroupN N tiles cycle fastest, so the workgroups in
// flight on one XCD share a few M and N tiles in its L2.
constexpr int kGroupN = 8;
struct TilePos {
  int m, n;
};
__device__ __forceinline__ TilePos tile_pos(int num_m, int num_n) {
  const int total = num_m * num_n;
  const int L = xcd_remap((int)blockIdx.x, total);
  const int per_group = kGroupN * num_m;
  const int group = L / per_group;
  const int first_n = group * kGroupN;
  const int size_n = min(num_n - first_n, kGroupN);
  const int in_group = L % per_group;
  return TilePos{in_group / size_n, first_n + in_group % size_n};
}

// 256 x 256 tile of C[M][N] += A[M][K] B[N][K]^T, A and B row-major with K
// contiguous (rows at a_rows / b_rows of `a_valid` / `b_valid` rows, element
// strides lda / ldb), K = kdim (a multiple of 64). Eight waves: wave w holds
// rows 128 (w / 4) .. +127 and columns 64 (w % 4) .. +63 as acc[i][j], the
// 32 x 32 block (i, j): lane l holds column 32 j + l % 32, rows 32 i + 8 (r / 4)
// + 4 (l / 32) + r % 4 of the wave's rows.
template <typename T>
__device__ __forceinline__ void gemm_nt_tile(f32x16 (&acc)[4][2], char* st0, char* st1, const T* A, int64_t lda,
                                             int a_valid, const T* B, int64_t ldb, int b_valid, int kdim,
                                             int w, int lane) {
  using Tile = LdsTile<T, kTile, kBK>;
  const int half = lane >> 5, l32 = lane & 31, wm = w >> 2, wn = w & 3;
  TileLoader<T, kTile, kBK, kThreads> la, lb;
  const uint32_t sa = (uint32_t)(lda * sizeof(T)), sb = (uint32_t)(ldb * sizeof(T));
  la.init(sa, w, lane);
  lb.init(sb, w, lane);
  RowReader<T, kBK> rrd;
  rrd.init(l32, half);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const int steps = kdim / kBK;
  auto fill = [&](char* st, int k) {
    la.issue(st, A + (int64_t)k * kBK, sa, a_valid);
    lb.issue(st + Tile::kBytes, B + (int64_t)k * kBK, sb, b_valid);
  };
  auto step = [&](const char* st) {
    const char* as = st;
    const char* bs = st + Tile::kBytes;
#pragma unroll
    for (int ss = 0; ss < kBK / 16; ++ss) {
      Frag<T> a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = rrd.read(as, 128 * wm + 32 * i, ss);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = rrd.read(bs, 64 * wn + 32 * j, ss);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mma(acc[i][j], a[i], b[j]);
    }
  };
  // odd step counts start in stage 1: the loop runs whole stage pairs
  fill(steps & 1 ? st1 : st0, 0);
  __syncthreads();
  int k = 0;
  if (steps & 1) {
    if (k + 1 < steps) fill(st0, k + 1);
    step(st1);
    __syncthreads();
    ++k;
  }
  for (; k < steps; k += 2) {
    if (k + 1 < steps) fill(st1, k + 1);
    step(st0);
    __syncthreads();
    if (k + 2 < steps) fill(st0, k + 2);
    step(st1);
    __syncthreads();
  }
}

// Transposing reads of the two 32-column blocks dt0, dt0 + 1 of a [K rows][D]
// LDS tile, k in the contiguous order RowReader gives the other operand
// (ColReader<T, D, true> for a run-time block index without an array
// indexed at run time).
template <typename T, int D>
struct ColPair {
  using Tile = LdsTile<T, 16, D>;
  int off[2][2];
  __device__ __forceinline__ void init(int lane, int dt0) {
    const int half = lane >> 5, r = lane & 15;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = 32 * (dt0 + j) + (lane & 16) + 4 * (r & 3);
      off[j][0] = Tile::elem_off(8 * half + (r >> 2), col);
      off[j][1] = Tile::elem_off(8 * half + 4 + (r >> 2), col);
    }
  }
  __device__ __forceinline__ Frag<T> read(const char* base, int kbase, int j) const {
    const char* p = base + kbase * Tile::kRowBytes;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + off[j][0]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + off[j][1]));
    short s8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    Frag<T> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = __builtin_bit_cast(T, s8[e]);
    return f;
  }
};

}  // namespace

// MODE kFwd: M = vocabulary (W rows), N = tokens (H rows); partial (max, sum)
// per (vocab tile, token) and the target logit.
// MODE kDz: M = tokens, N = the chunk's vocabulary; dz into the chunk buffer.
template <typename T, int MODE>
__global__ void __launch_bounds__(kThreads) ce_logits_kernel(CEArgs a) {
  using Tile = LdsTile<T, kTile, kBK>;
  __shared__ __attribute__((aligned(1024))) char st0[2 * Tile::kBytes];
  __shared__ __attribute__((aligned(1024))) char st1[2 * Tile::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int w = wave_uniform(tid >> 6), wm = w >> 2, wn = w & 3;
  const int vocab = MODE == kFwd ? a.vocab : a.vc;  // vocabulary rows this launch covers
  const int num_v = (vocab + kTile - 1) / kTile, num_t = (a.n + kTile - 1) / kTile;
  const int num_m = MODE == kFwd ? num_v : num_t, num_n = MODE == kFwd ? num_t : num_v;
  const TilePos tp = tile_pos(num_m, num_n);
  const int vt = MODE == kFwd ? tp.m : tp.n, tt = MODE == kFwd ? tp.n : tp.m;
  const T* H = static_cast<const T*>(a.h) + (int64_t)tt * kTile * a.hidden;
  const T* W = static_cast<const T*>(a.w) + ((int64_t)a.v0 + (int64_t)vt * kTile) * a.hidden;
  const int t_valid = min(kTile, a.n - tt * kTile), v_valid = min(kTile, vocab - vt * kTile);
  f32x16 acc[4][2];
  if constexpr (MODE == kFwd)
    gemm_nt_tile<T>(acc, st0, st1, W, a.hidden, v_valid, H, a.hidden, t_valid, a.hidden, w, lane);
  else
    gemm_nt_tile<T>(acc, st0, st1, H, a.hidden, t_valid, W, a.hidden, v_valid, a.hidden, w, lane);

  if constexpr (MODE == kFwd) {
    // lane's tokens: tt*256 + 64 wn + 32 j + l32; its rows (vocab) per block i:
    // vt*256 + 128 wm + 32 i + 8 (r/4) + 4 half + r % 4
    float* red = reinterpret_cast<float*>(st0);  // [2 wm][256 tokens] x (m2, s)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tl = 64 * wn + 32 * j + l32;  // token within the tile
      const int vrow0 = 128 * wm + 4 * half;  // vocab row (within the tile) of r = 0, block 0
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int vr = vrow0 + 32 * i + 8 * (r >> 2) + (r & 3);
          if (vr >= v_valid) acc[i][j][r] = -INFINITY;
          mx = fmaxf(mx, acc[i][j][r]);
        }
      mx = max_halves(mx) * kLog2e;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += fast_exp2(fmaf(acc[i][j][r], kLog2e, -mx));
      s = sum_halves(s);
      if (half == 0) {
        red[2 * (wm * kTile + tl)] = mx;
        red[2 * (wm * kTile + tl) + 1] = s;
      }
      // the target logit: the one lane holding (token, y) writes it
      const int t = tt * kTile + tl;
      const int yt = tl < t_valid ? a.targets[t] : -1;
      if (yt >= 0 && yt < a.vocab) {  // a target outside [0, V) is never written (stays NaN)
        const int y = yt - vt * kTile - vrow0;  // y relative to this lane's r = 0, block 0
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (y == 32 * i + 8 * (r >> 2) + (r & 3)) a.tgt[t] = acc[i][j][r];
      }
    }
    __syncthreads();
    if (tid < kTile && tid < t_valid) {  // combine the two vocabulary halves of each token
      const float m0 = red[2 * tid], s0 = red[2 * tid + 1];
      const float m1 = red[2 * (kTile + tid)], s1 = red[2 * (kTile + tid) + 1];
      const float m = fmaxf(m0, m1);
      const float sm = (m0 == -INFINITY ? 0.f : s0 * fast_exp2(m0 - m)) + (m1 == -INFINITY ? 0.f : s1 * fast_exp2(m1 - m));
      float2* part = reinterpret_cast<float2*>(a.part) + (int64_t)vt * a.n + tt * kTile + tid;
      *part = make_float2(m, sm);
    }
  } else {
    // lane's vocab column: vt*256 + 64 wn + 32 j + l32 (within the chunk); its
    // rows (tokens) per block i: tt*256 + 128 wm + 32 i + 8 (r/4) + 4 half + r % 4.
    // Per-token LSE*log2(e), g and y go through LDS first.
    float* lse2s = reinterpret_cast<float*>(st0);
    float* gs = lse2s + kTile;
    int* ys = reinterpret_cast<int*>(gs + kTile);
    if (tid < kTile) {
      const int t = tt * kTile + tid;
      const bool ok = tid < t_valid;
      lse2s[tid] = ok ? a.lse[t] * kLog2e : INFINITY;
      gs[tid] = ok ? a.dnll[t] : 0.f;
      ys[tid] = ok ? a.targets[t] - a.v0 - vt * kTile : -1;  // the target as a column of this tile
    }
    __syncthreads();
    T* dz = static_cast<T*>(a.dz);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int vl = 64 * wn + 32 * j + l32;  // vocab column within the tile
      const bool v_ok = vl < v_valid;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tl = 128 * wm + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
          const float p = fast_exp2(fmaf(acc[i][j][r], kLog2e, -lse2s[tl]));
          const float d = gs[tl] * (p - (ys[tl] == vl ? 1.f : 0.f));
          // columns from vc up to the stride hold zeros (read as K padding by ce_dh_kernel)
          if (tl < t_valid && vt * kTile + vl < a.ldz)
            dz[(int64_t)(tt * kTile + tl) * a.ldz + vt * kTile + vl] = from_f32<T>(v_ok ? d : 0.f);
        }
    }
  }
}

// dH[t][d] (+)= sum over the chunk's vocabulary of dz[t][v] W[v0 + v][d]:
// M = tokens (dz rows), N = hidden (W columns, read transposed from W rows),
// K = the chunk's vocabulary. `first`: no earlier chunk (store); `last`: write
// dH in the I/O type (else the fp32 accumulator).
template <typename T>
__global__ void __launch_bounds__(kThreads) ce_dh_kernel(CEArgs a, int first, int last) {
  using ATile = LdsTile<T, kTile, kBK>;  // dz: 256 tokens x 64 vocab
  using BTile = LdsTile<T, kBK, kTile>;  // W: 64 vocab x 256 hidden
  static_assert(ATile::kBytes == BTile::kBytes, "equal halves");
  __shared__ __attribute__((aligned(1024))) char st0[2 * ATile::kBytes];
  __shared__ __attribute__((aligned(1024))) char st1[2 * ATile::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int w = wave_uniform(tid >> 6), wm = w >> 2, wn = w & 3;
  const int num_t = (a.n + kTile - 1) / kTile, num_d = a.hidden / kTile;
  const TilePos tp = tile_pos(num_t, num_d);
  const int tt = tp.m, dtile = tp.n;
  const int t_valid = min(kTile, a.n - tt * kTile);
  const T* DZ = static_cast<const T*>(a.dz) + (int64_t)tt * kTile * a.ldz;
  const T* W = static_cast<const T*>(a.w) + (int64_t)a.v0 * a.hidden + dtile * kTile;
  TileLoader<T, kTile, kBK, kThreads> la;
  TileLoader<T, kBK, kTile, kThreads> lb;
  const uint32_t sa = (uint32_t)(a.ldz * (int64_t)sizeof(T)), sb = (uint32_t)(a.hidden * (int64_t)sizeof(T));
  la.init(sa, w, lane);
  lb.init(sb, w, lane);
  RowReader<T, kBK> rrd;
  rrd.init(l32, half);
  ColPair<T, kTile> crd;
  crd.init(lane, 2 * wn);
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const int steps = a.ldz / kBK;
  // the chunk's padding columns of dz hold zeros and the matching W rows (past
  // the chunk) arrive as zeros
  auto fill = [&](char* st, int k) {
    la.issue(st, DZ + (int64_t)k * kBK, sa, t_valid);
    lb.issue(st + ATile::kBytes, W + (int64_t)k * kBK * a.hidden, sb, min(kBK, a.vc - k * kBK));
  };
  auto step = [&](const char* st) {
    const char* as = st;
    const char* bs = st + ATile::kBytes;
#pragma unroll
    for (int ss = 0; ss < kBK / 16; ++ss) {
      Frag<T> x[4], y[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = rrd.read(as, 128 * wm + 32 * i, ss);
#pragma unroll
      for (int j = 0; j < 2; ++j) y[j] = crd.read(bs, 16 * ss, j);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mma(acc[i][j], x[i], y[j]);
    }
  };
  fill(steps & 1 ? st1 : st0, 0);
  __syncthreads();
  int k = 0;
  if (steps & 1) {
    if (k + 1 < steps) fill(st0, k + 1);
    step(st1);
    __syncthreads();
    ++k;
  }
  for (; k < steps; k += 2) {
    if (k + 1 < steps) fill(st1, k + 1);
    step(st0);
    __syncthreads();
    if (k + 2 < steps) fill(st0, k + 2);
    step(st1);
    __syncthreads();
  }
  // lane's hidden column: dtile*256 + 64 wn + 32 j + l32; rows (tokens) per
  // block i: tt*256 + 128 wm + 32 i + 8 (r/4) + 4 half + r % 4
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tl = 128 * wm + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
      if (tl >= t_valid) continue;
      const int64_t row = (int64_t)(tt * kTile + tl) * a.hidden + dtile * kTile + 64 * wn + l32;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float v = acc[i][j][r];
        if (!first) v += a.dh32[row + 32 * j];
        if (last) static_cast<T*>(a.dh)[row + 32 * j] = from_f32<T>(v);
        else a.dh32[row + 32 * j] = v;
      }
    }
}

// Per token: fold the per-tile (max, sum) partials into LSE (natural log) and
// the loss. A block takes 16 tokens; its 16 thread groups split the vocabulary
// tiles (reads of 16 consecutive tokens stay contiguous) and combine through
// LDS. A target outside [0, V) was never found: its logit stays NaN.
constexpr int kRedTok = 16, kRedGrp = 16;
__global__ void __launch_bounds__(kRedTok * kRedGrp) ce_reduce_kernel(CEArgs a) {
  __shared__ float2 acc[kRedGrp][kRedTok];
  const int tl = threadIdx.x % kRedTok, grp = threadIdx.x / kRedTok;
  const int t = blockIdx.x * kRedTok + tl;
  const int num_v = (a.vocab + kTile - 1) / kTile;
  float m = -INFINITY, s = 0.f;
  if (t < a.n) {
    const float2* part = reinterpret_cast<const float2*>(a.part) + t;
    for (int v = grp; v < num_v; v += kRedGrp) {
      const float2 p = part[(int64_t)v * a.n];
      if (p.x == -INFINITY) continue;
      const float mn = fmaxf(m, p.x);
      s = (m == -INFINITY ? 0.f : s * fast_exp2(m - mn)) + p.y * fast_exp2(p.x - mn);
      m = mn;
    }
  }
  acc[grp][tl] = make_float2(m, s);
  __syncthreads();
  if (grp == 0 && t < a.n) {
    float mt = -INFINITY;
#pragma unroll
    for (int g = 0; g < kRedGrp; ++g) mt = fmaxf(mt, acc[g][tl].x);
    float st = 0.f;
#pragma unroll
    for (int g = 0; g < kRedGrp; ++g)
      if (acc[g][tl].x != -INFINITY) st += acc[g][tl].y * fast_exp2(acc[g][tl].x - mt);
    const float lse = (mt + fast_log2(st)) * kLn2;
    a.out_lse[t] = lse;
    a.nll[t] = lse - a.tgt[t];
  }
}

// the target logits start as NaN (a target outside [0, V) is never found)
__global__ void __launch_bounds__(256) ce_fill_nan_kernel(float* p, int n) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < n) p[t] = NAN;
}

// ------------------------------------------------------------ launchers

int ce_vocab_chunk(int vocab) {
  const int cap = 16384;  // dz chunk: n x 16384 elements
  const int v = (vocab + kTile - 1) / kTile * kTile;
  return v < cap ? v : cap;
}

template <typename T>
static hipError_t ce_fwd_t(const CEArgs& a0, hipStream_t st) {
  CEArgs a = a0;
  a.v0 = 0;
  a.vc = a.vocab;
  hipLaunchKernelGGL(ce_fill_nan_kernel, dim3((unsigned)((a.n + 255) / 256)), dim3(256), 0, st, a.tgt, a.n);
  const int64_t grid = (int64_t)((a.vocab + kTile - 1) / kTile) * ((a.n + kTile - 1) / kTile);
  hipLaunchKernelGGL((ce_logits_kernel<T, kFwd>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL(ce_reduce_kernel, dim3((unsigned)((a.n + kRedTok - 1) / kRedTok)), dim3(kRedTok * kRedGrp), 0,
                     st, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t ce_bwd_t(const CEArgs& a0, hipStream_t st) {
  CEArgs a = a0;
  const int chunk = ce_vocab_chunk(a.vocab);
  const int nt = (a.n + kTile - 1) / kTile;
  for (int v0 = 0; v0 < a.vocab; v0 += chunk) {
    a.v0 = v0;
    a.vc = min(chunk, a.vocab - v0);
    a.ldz = (a.vc + kBK - 1) / kBK * kBK;
    const int64_t g1 = (int64_t)((a.vc + kTile - 1) / kTile) * nt;
    hipLaunchKernelGGL((ce_logits_kernel<T, kDz>), dim3((unsigned)g1), dim3(kThreads), 0, st, a);
    const int64_t g2 = (int64_t)nt * (a.hidden / kTile);
    hipLaunchKernelGGL((ce_dh_kernel<T>), dim3((unsigned)g2), dim3(kThreads), 0, st, a, v0 == 0 ? 1 : 0,
                       v0 + chunk >= a.vocab ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_ce_fwd(int dtype, const CEArgs& a, hipStream_t st) {
  if (a.n == 0) return hipSuccess;
  if (dtype == 1) return ce_fwd_t<bf16>(a, st);
  if (dtype == 2) return ce_fwd_t<fp16>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_ce_bwd(int dtype, const CEArgs& a, hipStream_t st) {
  if (a.n == 0) return hipSuccess;
  if (dtype == 1) return ce_bwd_t<bf16>(a, st);
  if (dtype == 2) return ce_bwd_t<fp16>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace swa
