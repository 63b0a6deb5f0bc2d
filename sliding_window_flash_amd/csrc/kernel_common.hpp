// Shared device building blocks for the gfx950 attention kernels.
//
// MFMA: every contraction uses the 32x32 result tile. bf16 and fp16 operands
// use v_mfma_f32_32x32x16_{bf16,f16} (one instruction per 16-deep step, the
// same lane layout); fp32 operands use eight v_mfma_f32_32x32x2_f32 (true
// fp32, no reduced-precision mode).
//
// Lane layouts (64 lanes; l32 = lane % 32, half = lane / 32):
//   A operand (M x 16): lane holds row l32, 8 contraction elements
//   B operand (16 x N): lane holds column l32, 8 contraction elements
//   result (32 x 32 fp32, 16 registers): lane holds column l32; register r is
//   row 8*(r/4) + 4*half + r%4.
// Which 8 contraction indices a lane holds is free as long as A and B agree.
// A result tile read back as an operand (P or dS) gives, for its 16-deep step
// u in {0, 1}, the indices 16u + 4*half + {0..3} and 16u + 8 + 4*half + {0..3}
// (registers 8u..8u+7). Every operand read along the rows of an LDS tile
// (col_frag) therefore fetches those same indices.
//
// LDS tiles hold rows of head_dim elements, unpadded, with 16-byte chunks
// XOR-swizzled per row so that (a) 16 lanes reading 16 consecutive rows at the
// same chunk and (b) the 4-row x 4-chunk blocks of a transposing read both
// touch distinct banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sched.hpp"

namespace swa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 fp16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- operand fragments -------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<fp16> { f16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void mma(f32x16& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& c, const Frag<fp16>& a, const Frag<fp16>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[j], b.v[j], c, 0, 0, 0);
}

// Registers 8u..8u+7 of a result tile as an operand fragment (P or dS).
template <typename T> __device__ __forceinline__ Frag<T> acc_frag(const f32x16& c, int u);
template <> __device__ __forceinline__ Frag<bf16> acc_frag<bf16>(const f32x16& c, int u) {
  Frag<bf16> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = (bf16)c[8 * u + j];  // round to nearest even
  return f;
}
template <> __device__ __forceinline__ Frag<fp16> acc_frag<fp16>(const f32x16& c, int u) {
  Frag<fp16> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = (fp16)c[8 * u + j];  // round to nearest even
  return f;
}
template <> __device__ __forceinline__ Frag<float> acc_frag<float>(const f32x16& c, int u) {
  Frag<float> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = c[8 * u + j];
  return f;
}

// ---- element conversion ---------------------------------------------------
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(fp16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ fp16 from_f32<fp16>(float x) { return (fp16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// ---- swizzled LDS tile ------------------------------------------------------
// ROWS x D elements of T; rows are D*sizeof(T) bytes (a multiple of 16).
template <typename T, int ROWS, int D> struct LdsTile {
  static constexpr int kChunks = D * (int)sizeof(T) / 16;   // 16-byte chunks per row
  static constexpr int kRowBytes = kChunks * 16;
  static constexpr int kBytes = ROWS * kRowBytes;
  static constexpr int kElemsPerChunk = 16 / (int)sizeof(T);
  static_assert(kChunks == 8 || kChunks >= 16, "row must be 128 bytes or >= 256 bytes");

  __device__ static __forceinline__ int swz(int r) {
    return kChunks >= 16 ? (4 * (r & 3) + ((r >> 2) & 3)) : ((r >> 1) & 7);
  }
  // byte offset of chunk c of row r
  __device__ static __forceinline__ int chunk_off(int r, int c) {
    return r * kRowBytes + ((c ^ swz(r)) << 4);
  }
  // byte offset of element e of row r
  __device__ static __forceinline__ int elem_off(int r, int e) {
    const int byte = e * (int)sizeof(T);
    return chunk_off(r, byte >> 4) + (byte & 15);
  }
};

// Operand fragment read along a row: row `row`, contraction elements
// [8*k8, 8*k8+8) of that row.
template <typename T, int ROWS, int D>
__device__ __forceinline__ Frag<T> row_frag(const char* lds, int row, int k8) {
  using Tile = LdsTile<T, ROWS, D>;
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(lds + Tile::chunk_off(row, k8));
    f.v = __builtin_bit_cast(decltype(f.v), raw);
  } else {
    // float vectors, not bit casts of u32x4 elements: the latter is folded to
    // element 0 by this compiler.
    const f32x4 a = *reinterpret_cast<const f32x4*>(lds + Tile::chunk_off(row, 2 * k8));
    const f32x4 b = *reinterpret_cast<const f32x4*>(lds + Tile::chunk_off(row, 2 * k8 + 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f.v[j] = a[j];
      f.v[4 + j] = b[j];
    }
  }
  return f;
}

// Operand fragment read down a column: the lane's column is nbase + lane%32;
// the contraction runs over rows kbase + (the 8 indices listed at the top for
// lane half lane/32). kbase is a multiple of 16.
template <typename T, int ROWS, int D>
__device__ __forceinline__ Frag<T> col_frag(const char* lds, int kbase, int nbase, int lane) {
  using Tile = LdsTile<T, ROWS, D>;
  const int half = lane >> 5;
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    // ds_read_tr16_b64: in each 16-lane group, lane i receives element i%4 of
    // the 8 bytes addressed by lanes 4e + i/4 (e = 0..3). Lane r of the group
    // addresses row k0 + r/4 at columns n0 + 4*(r%4) .. +3, so lane i gets rows
    // k0..k0+3 of column n0 + i.
    const int r = lane & 15;
    const int n0 = nbase + (lane & 16);
    const int col = n0 + 4 * (r & 3);
    i16x4 lo, hi;
    {
      const int row = kbase + 4 * half + (r >> 2);
      lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(lds + Tile::elem_off(row, col)));
    }
    {
      const int row = kbase + 8 + 4 * half + (r >> 2);
      hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(lds + Tile::elem_off(row, col)));
    }
    short s8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = __builtin_bit_cast(T, s8[j]);
  } else {
    const int n = nbase + (lane & 31);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = kbase + (j < 4 ? 4 * half + j : 8 + 4 * half + (j - 4));
      f.v[j] = *reinterpret_cast<const float*>(lds + Tile::elem_off(row, n));
    }
  }
  return f;
}

// Row and column fragment readers with per-lane offsets computed once. The
// swizzle depends only on row % 16, so for a row block starting at a multiple
// of 16 rows every address is (block start x row bytes) + a per-lane offset:
// with the block start and the LDS stage known at compile time, each read is
// one register plus an immediate. In rows of 16 chunks or more the swizzle
// changes only the low 4 bits of a chunk index, so the offsets repeat every
// 16 chunks (256 bytes) apart: a reader keeps one period of them and adds the
// rest as an immediate.
template <typename T, int D>
struct RowReader {
  using Tile = LdsTile<T, 16, D>;
  static constexpr int kSteps = D / 16;
  static constexpr int kParts = sizeof(T) == 2 ? 1 : 2;  // 16-byte chunks per fragment
  // steps per 16 chunks (a step advances 2 kParts chunks)
  static constexpr int kPeriod = Tile::kChunks >= 16 && kSteps > 8 / kParts ? 8 / kParts : kSteps;
  int off[kPeriod][kParts];
  __device__ __forceinline__ void init(int l32, int half) {
#pragma unroll
    for (int ss = 0; ss < kPeriod; ++ss)
#pragma unroll
      for (int q = 0; q < kParts; ++q) off[ss][q] = Tile::chunk_off(l32, kParts * (2 * ss + half) + q);
  }
  // same as row_frag(base, row16 + lane%32, 2*ss + half); row16 % 16 == 0
  __device__ __forceinline__ Frag<T> read(const char* base, int row16, int ss) const {
    const char* p = base + row16 * Tile::kRowBytes + (ss / kPeriod) * 256;
    const int si = ss % kPeriod;
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(p + off[si][0]);
      f.v = __builtin_bit_cast(decltype(f.v), raw);
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(p + off[si][0]);
      const f32x4 b = *reinterpret_cast<const f32x4*>(p + off[si][1]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f.v[j] = a[j];
        f.v[4 + j] = b[j];
      }
    }
    return f;
  }
};

template <typename T, int D>
struct ColReader {
  using Tile = LdsTile<T, 16, D>;
  static constexpr int kBlocks = D / 32;
  static constexpr int kParts = sizeof(T) == 2 ? 2 : 8;  // transposing reads / scalar reads
  // 32-column blocks per 16 chunks (a block spans 32 * sizeof(T) / 16 chunks)
  static constexpr int kPer16 = 16 / (2 * (int)sizeof(T));
  static constexpr int kPeriod = Tile::kChunks >= 16 && kBlocks > kPer16 ? kPer16 : kBlocks;
  int off[kPeriod][kParts];
  __device__ __forceinline__ void init(int lane) {
    const int half = lane >> 5;
#pragma unroll
    for (int dt = 0; dt < kPeriod; ++dt) {
      if constexpr (sizeof(T) == 2) {
        const int r = lane & 15;
        const int col = 32 * dt + (lane & 16) + 4 * (r & 3);
        off[dt][0] = Tile::elem_off(4 * half + (r >> 2), col);
        off[dt][1] = Tile::elem_off(8 + 4 * half + (r >> 2), col);
      } else {
        const int n = 32 * dt + (lane & 31);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          off[dt][j] = Tile::elem_off(j < 4 ? 4 * half + j : 8 + 4 * half + (j - 4), n);
      }
    }
  }
  // same as col_frag(base, kbase, 32*dt, lane); kbase % 16 == 0
  __device__ __forceinline__ Frag<T> read(const char* base, int kbase, int dt) const {
    const char* p = base + kbase * Tile::kRowBytes + (dt / kPeriod) * 256;
    const int di = dt % kPeriod;
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(p + off[di][0]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(p + off[di][1]));
      short s8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int j = 0; j < 8; ++j) f.v[j] = __builtin_bit_cast(T, s8[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) f.v[j] = *reinterpret_cast<const float*>(p + off[di][j]);
    }
    return f;
  }
};

// Raw buffer resource over [base, base + bytes): loads through it are
// range-checked on their byte offset, so an offset at or past `bytes` returns
// zero and touches no memory. Word 3 is the gfx9 raw-buffer format word
// (32-bit data format, no swizzle, no stride).
constexpr int kBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

// The LDS address of a generic pointer into shared memory: the generic
// aperture keeps the LDS offset in the low 32 bits. Taking them directly,
// rather than casting the pointer, spares the null check that a generic to
// LDS cast carries (a compare against the aperture base per call).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wint-to-void-pointer-cast"
__device__ __forceinline__ __attribute__((address_space(3))) void* lds_addr(const void* p) {
  return (__attribute__((address_space(3))) void*)(uint32_t)(uintptr_t)p;
}
#pragma clang diagnostic pop

// One buffer load per lane into LDS, 16 or 4 bytes: lane l's data lands at
// lds + l * bytes (lds wave-uniform).
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rsrc, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_addr(lds), 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void buffer_to_lds4(__amdgpu_buffer_rsrc_t rsrc, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_addr(lds), 4, voff, 0, 0, 0);
}

// Direct global -> LDS copy of a ROWS x D tile into the swizzled layout
// (buffer_load_dwordx4 ... lds: each wave instruction writes 64 consecutive
// 16-byte LDS slots; the lane of physical slot (row, pc) fetches logical chunk
// pc ^ swz(row) of that row). The per-lane byte offsets are fixed for a
// kernel, so a tile costs one descriptor and kPerWave loads per wave. Rows at
// or past `valid` lie outside the descriptor's range and arrive as zeros; no
// address outside the sequence's rows is read. No registers hold the data: it
// lands in LDS asynchronously, and the compiler waits for it (vmcnt) before
// the next barrier. Buffer loads, unlike the flat-segment global_load_lds,
// leave the compiler's LDS read counting exact, so reads can run ahead of the
// MFMAs that consume them.
template <typename T, int ROWS, int D, int NT>
struct TileLoader {
  using Tile = LdsTile<T, ROWS, D>;
  static constexpr int kInstr = ROWS * Tile::kChunks / 64;
  static constexpr int kPerWave = kInstr / (NT / 64);
  static_assert(kInstr % (NT / 64) == 0, "tile must split evenly over the waves");
  uint32_t off[kPerWave];  // byte offset of this lane's chunk from the tile's first row
  int lds0;                // byte offset of this wave's first LDS slot (wave-uniform)
  // stride_bytes: bytes between consecutive rows; ROWS * stride_bytes < 2^31
  __device__ __forceinline__ void init(uint32_t stride_bytes, int wave, int lane) {
    lds0 = wave * kPerWave * 1024;
#pragma unroll
    for (int e = 0; e < kPerWave; ++e) {
      const int slot = (wave * kPerWave + e) * 64 + lane;
      const int row = slot / Tile::kChunks, pc = slot % Tile::kChunks;
      off[e] = (uint32_t)row * stride_bytes + (uint32_t)(pc ^ Tile::swz(row)) * 16u;
    }
  }
  // src: first element of the tile's first row; valid in [1, ROWS] rows exist
  __device__ __forceinline__ void issue(char* lds, const T* src, uint32_t stride_bytes, int valid) const {
    const __amdgpu_buffer_rsrc_t rsrc = buffer_rsrc(src, (uint32_t)valid * stride_bytes);
#pragma unroll
    for (int e = 0; e < kPerWave; ++e) buffer_to_lds16(rsrc, lds + lds0 + e * 1024, off[e]);
  }
};

// Fragment straight from global memory: 8 consecutive elements at p.
template <typename T> __device__ __forceinline__ Frag<T> global_frag(const T* __restrict__ p) {
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(p);
    f.v = __builtin_bit_cast(decltype(f.v), raw);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f.v[j] = a[j];
      f.v[4 + j] = b[j];
    }
  }
  return f;
}
template <typename T> __device__ __forceinline__ Frag<T> zero_frag() {
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = (T)0.0f;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = 0.0f;
  }
  return f;
}

// A wave-uniform value the compiler can keep in a scalar register.
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Sum of the 8 values of a 16-bit fragment added to `acc` (four v_dot2
// against (1, 1); products by one are exact, the sum is accumulated in fp32).
__device__ __forceinline__ float frag_sum(const Frag<fp16>& f, float acc) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 one = {(fp16)1.0f, (fp16)1.0f};
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(f.v, f.v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(f.v, f.v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(f.v, f.v, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2(__builtin_shufflevector(f.v, f.v, 6, 7), one, acc, false);
}
__device__ __forceinline__ float frag_sum(const Frag<bf16>& f, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f.v, f.v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f.v, f.v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f.v, f.v, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f.v, f.v, 6, 7), one, acc, false);
}

// Reductions over lanes l and l ^ 32 (the two halves of a wave hold the two
// 8-row halves of each score column), left in every lane. One
// v_permlane32_swap with both operands x yields, in every lane, the lower
// half's value (first result) and the upper half's (second result), so no LDS
// round trip is needed.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return a > b ? a : b;
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Kernel argument block shared by all launches.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  const int32_t* cu_q;
  const int32_t* cu_k;
  void* out_o;
  float* out_lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // -D = -rowsum(dO * O), [heads_q, total_q] (negated: the dP accumulators start from it)
  float* lse2;   // LSE * log2(e) (+inf where LSE = -inf), [heads_q, total_q]
  // dK/dV with the group's query heads split over kv_split workgroups per key
  // tile (kv_split > 1 when there are too few key tiles to fill the GPU):
  // fp32 partial sums [kv_split][dK, dV][total_k, heads_kv, head_dim], added
  // up by a second launch
  float* dkv_part;
  int32_t kv_split;
  // optional mask combined with the window: row t (packed query token) is
  // mask_words uint32 words, bit j % 32 of word j / 32 allows key j of the
  // token's sequence; nullptr = no mask
  const uint32_t* mask;
  int64_t mask_words;
  // optional per-block ranges of the mask's allowed bits (mask_range_kernel):
  // [batch][nrb][2] first/last 32-key block per 32-row block, then
  // [batch][nkb32][2] first/last 32-row block per 32-key block; nullptr = none
  const int32_t* mask_ranges;
  int32_t batch, heads_q, heads_kv, total_q, total_k, max_seqlen_q, max_seqlen_k;
  int32_t window, causal;
  float scale;
  // Launch-invariant parts of the launch-id decode, set by the launchers
  // (with_decode): query-major items (forward, dQ) take 2^q_hw_log2 query
  // heads of a group of q_grp, in q_nch chunks, and q_rows rows, in q_nqb row
  // blocks per sequence (q_items in all); key-major items (dK/dV) take a key
  // tile of 128 (k_nkb per sequence) and k_hpp of the group's query heads
  // (k_items in all). The divisions of the decode use the multipliers.
  int32_t q_grp, q_hw_log2, q_nch, q_rows, q_nqb, q_items, k_nkb, k_hpp, k_items;
  FastDiv div_nch, div_nqb, div_batch, div_nkb, div_split;
};

}  // namespace swa
