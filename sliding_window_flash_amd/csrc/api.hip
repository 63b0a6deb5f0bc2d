// C ABI of the attention library: argument checks, then launches on the
// caller's stream. Declarations and the contract are in include/swa_attn.h.
#include <math.h>
#include <stdint.h>

#include "../../include/swa_attn.h"
#include "../../include/swa_ce.h"
#include "ce_launch.hpp"
#include "launch.hpp"
#include "sched.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// A tensor pointer may be NULL only when the tensor has no elements.
attn_status_t check_tensor(const void* ptr, int64_t elems, bool vec16) {
  if (elems == 0) return ATTN_OK;
  if (ptr == nullptr) return ATTN_ERR_NULL;
  if (vec16 ? !aligned16(ptr) : !aligned4(ptr)) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

swa::AttnArgs base_args(const attn_params_t* p) {
  swa::AttnArgs a{};
  a.batch = p->batch;
  a.heads_q = p->heads_q;
  a.heads_kv = p->heads_kv;
  a.total_q = p->total_q;
  a.total_k = p->total_k;
  a.max_seqlen_q = p->max_seqlen_q;
  a.max_seqlen_k = p->max_seqlen_k;
  a.window = p->window;
  a.causal = p->causal;
  a.scale = p->scale;
  a.kv_split = 1;
  return a;
}

// a * b * c <= INT32_MAX for non-negative factors, without overflowing
bool fits_i32(int64_t a, int64_t b, int64_t c) {
  if (a == 0 || b == 0 || c == 0) return true;
  return a <= INT32_MAX / b && a * b <= INT32_MAX / c;
}

int64_t q_elems(const attn_params_t* p) { return (int64_t)p->total_q * p->heads_q * p->head_dim; }
int64_t k_elems(const attn_params_t* p) { return (int64_t)p->total_k * p->heads_kv * p->head_dim; }

}  // namespace

extern "C" {

attn_status_t attn_check_params(const attn_params_t* p) {
  if (p == nullptr) return ATTN_ERR_NULL;
  if (p->batch < 1 || p->heads_q < 1 || p->heads_kv < 1 || p->heads_q % p->heads_kv != 0 ||
      p->total_q < 0 || p->total_k < 0 || p->max_seqlen_q < 0 || p->max_seqlen_k < 0 ||
      p->max_seqlen_q > p->total_q || p->max_seqlen_k > p->total_k)
    return ATTN_ERR_SHAPE;
  if (p->window < 1) return ATTN_ERR_WINDOW;
  if (p->dtype != ATTN_F32 && p->dtype != ATTN_BF16 && p->dtype != ATTN_F16) return ATTN_ERR_UNSUPPORTED;
  // head_dim 256 and 512 are built for the 16-bit types (fp32 there would need
  // twice the registers and LDS of the 16-bit kernels)
  if (p->head_dim != 64 && p->head_dim != 128 &&
      !((p->head_dim == 256 || p->head_dim == 512) && p->dtype != ATTN_F32))
    return ATTN_ERR_UNSUPPORTED;
  if (p->causal != 0 && p->causal != 1) return ATTN_ERR_UNSUPPORTED;
  // a two-sided window (no causal mask) shorter than the longer of the two
  // lengths forms p + window - 1 in 32 bits in the kernels' masks
  {
    const int32_t lmax = p->max_seqlen_q > p->max_seqlen_k ? p->max_seqlen_q : p->max_seqlen_k;
    if (p->causal == 0 && p->window < lmax && lmax > (1 << 30)) return ATTN_ERR_UNSUPPORTED;
  }
  // the kernels fold the scale into exp2 arguments and take row maxima on raw
  // scores, which needs a positive scale
  if (!(p->scale > 0.f) || !isfinite(p->scale)) return ATTN_ERR_UNSUPPORTED;
  // tile loads address a 128-row tile with 32-bit byte offsets: 128 rows x
  // heads x head_dim x element bytes must stay below 2^31
  const int64_t esize = p->dtype == ATTN_F32 ? 4 : 2;
  if (p->heads_q > 16384 || 128 * (int64_t)p->heads_q * p->head_dim * esize >= (int64_t(1) << 31))
    return ATTN_ERR_SHAPE;
  // packed element counts must stay addressable
  if ((int64_t)p->total_q * p->heads_q > INT32_MAX || (int64_t)p->total_k * p->heads_kv > INT32_MAX)
    return ATTN_ERR_SHAPE;
  // the kernels take their work item from a 32-bit launch id: query-major
  // grids have at most ceil(max_seqlen_q / 32) x heads_q x batch items, key-major
  // ones at most ceil(max_seqlen_k / 64) x heads_kv x batch
  if (!fits_i32(((int64_t)p->max_seqlen_q + 31) / 32, p->heads_q, p->batch) ||
      !fits_i32(((int64_t)p->max_seqlen_k + 63) / 64, p->heads_kv, p->batch))
    return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

static attn_status_t check_mask(const attn_params_t* p, const attn_mask_t* m) {
  if (m == nullptr) return ATTN_ERR_NULL;
  if (m->row_words < 1 || m->row_words % 4 != 0 || m->row_words < ((int64_t)p->max_seqlen_k + 31) / 32)
    return ATTN_ERR_SHAPE;
  // a 64-row mask tile is addressed with 32-bit byte offsets: 64 rows x
  // row_words x 4 bytes must stay below 2^32
  if (m->row_words >= (1 << 24)) return ATTN_ERR_UNSUPPORTED;
  if (m->ranges != nullptr && !aligned4(m->ranges)) return ATTN_ERR_ALIGN;
  return check_tensor(m->bits, (int64_t)p->total_q * m->row_words, true);
}

static size_t ranges_entries(const attn_params_t* p) {
  return 2 * (size_t)p->batch * (size_t)(((int64_t)p->max_seqlen_q + 31) / 32 + ((int64_t)p->max_seqlen_k + 31) / 32);
}

static attn_status_t fwd_impl(const attn_params_t* p, const attn_mask_t* mask, const void* q,
                              const void* k, const void* v, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, void* o, float* lse, void* stream) {
  attn_status_t s = attn_check_params(p);
  if (s != ATTN_OK) return s;
  if (mask != nullptr && (s = check_mask(p, mask)) != ATTN_OK) return s;
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return ATTN_ERR_NULL;
  if (!aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k)) return ATTN_ERR_ALIGN;
  const int64_t nq = q_elems(p), nk = k_elems(p);
  if ((s = check_tensor(q, nq, true)) != ATTN_OK) return s;
  if ((s = check_tensor(k, nk, true)) != ATTN_OK) return s;
  if ((s = check_tensor(v, nk, true)) != ATTN_OK) return s;
  if ((s = check_tensor(o, nq, true)) != ATTN_OK) return s;
  if ((s = check_tensor(lse, (int64_t)p->total_q * p->heads_q, false)) != ATTN_OK) return s;
  swa::AttnArgs a = base_args(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.out_o = o;
  a.out_lse = lse;
  if (mask != nullptr) {
    a.mask = mask->bits;
    a.mask_words = mask->row_words;
    a.mask_ranges = mask->ranges;
  }
  if (swa::launch_fwd(p->dtype, p->head_dim, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status_t attn_fwd(const attn_params_t* p, const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* o,
                       float* lse, void* stream) {
  return fwd_impl(p, nullptr, q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, stream);
}

size_t attn_mask_ranges_bytes(const attn_params_t* p) {
  if (attn_check_params(p) != ATTN_OK) return 0;
  return ranges_entries(p) * sizeof(int32_t);
}

attn_status_t attn_mask_ranges(const attn_params_t* p, const attn_mask_t* mask, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, int32_t* ranges, void* stream) {
  attn_status_t s = attn_check_params(p);
  if (s != ATTN_OK) return s;
  if ((s = check_mask(p, mask)) != ATTN_OK) return s;
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return ATTN_ERR_NULL;
  if (!aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k)) return ATTN_ERR_ALIGN;
  if ((s = check_tensor(ranges, (int64_t)ranges_entries(p), false)) != ATTN_OK) return s;
  swa::AttnArgs a = base_args(p);
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.mask = mask->bits;
  a.mask_words = mask->row_words;
  if (swa::launch_mask_ranges(a, ranges, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status_t attn_fwd_masked(const attn_params_t* p, const attn_mask_t* mask, const void* q,
                              const void* k, const void* v, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, void* o, float* lse, void* stream) {
  attn_status_t s = attn_check_params(p);
  if (s != ATTN_OK) return s;
  if (mask == nullptr) return ATTN_ERR_NULL;
  return fwd_impl(p, mask, q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, stream);
}

// Workspace: D [heads_q, total_q] fp32, then LSE*log2(e) [heads_q, total_q]
// fp32, each 256-byte aligned; then, when the dK/dV launch splits each KV
// group's query heads over `split` workgroups (too few key tiles to fill the
// GPU), the parts' fp32 partial dK and dV [split][2][total_k, heads_kv,
// head_dim].
static size_t ws_array_bytes(const attn_params_t* p) {
  const size_t n = (size_t)p->heads_q * (size_t)p->total_q * sizeof(float);
  return round_up(n > 0 ? n : 1, 256);
}

static int dkdv_split(const attn_params_t* p) {
  return swa::dkdv_split(p->dtype, p->head_dim, p->heads_q, p->heads_kv, p->batch, p->max_seqlen_k);
}

static size_t ws_bytes(const attn_params_t* p, int split) {
  size_t b = 2 * ws_array_bytes(p);
  if (split > 1) b += (size_t)split * 2 * (size_t)p->total_k * p->heads_kv * p->head_dim * sizeof(float);
  return b;
}

size_t attn_bwd_workspace_bytes(const attn_params_t* p) {
  if (attn_check_params(p) != ATTN_OK) return 0;
  return ws_bytes(p, dkdv_split(p));
}

static attn_status_t bwd_impl(const attn_params_t* p, const attn_mask_t* mask, int32_t stages,
                              const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes, void* stream,
                              bool use_scratch = false) {
  attn_status_t s = attn_check_params(p);
  if (s != ATTN_OK) return s;
  if (mask != nullptr && (s = check_mask(p, mask)) != ATTN_OK) return s;
  if (stages <= 0 || (stages & ~ATTN_BWD_ALL) != 0) return ATTN_ERR_SHAPE;
  const bool st_delta = stages & ATTN_BWD_DELTA, st_dq = stages & ATTN_BWD_DQ,
             st_dkdv = stages & ATTN_BWD_DKDV;
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return ATTN_ERR_NULL;
  if (!aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k)) return ATTN_ERR_ALIGN;
  const int64_t nq = q_elems(p), nk = k_elems(p), nrow = (int64_t)p->total_q * p->heads_q;
  if (st_dq || st_dkdv) {
    if ((s = check_tensor(q, nq, true)) != ATTN_OK) return s;
    if ((s = check_tensor(k, nk, true)) != ATTN_OK) return s;
    if ((s = check_tensor(v, nk, true)) != ATTN_OK) return s;
  }
  // O and LSE are read by the D preprocess and by dQ, which forms D itself
  if ((st_delta || st_dq) && (s = check_tensor(lse, nrow, false)) != ATTN_OK) return s;
  if ((st_delta || st_dq) && (s = check_tensor(o, nq, true)) != ATTN_OK) return s;
  if ((s = check_tensor(dout, nq, true)) != ATTN_OK) return s;
  if (st_dq && (s = check_tensor(dq, nq, true)) != ATTN_OK) return s;
  if (st_dkdv) {
    if ((s = check_tensor(dk, nk, true)) != ATTN_OK) return s;
    if ((s = check_tensor(dv, nk, true)) != ATTN_OK) return s;
  }
  // the no-allocation entry point keeps D and LSE*log2(e) only: no head split
  const int split = use_scratch ? 1 : dkdv_split(p);
  if (use_scratch) {
    // the library's fixed per-GPU array instead of a caller workspace: checked
    // against its size before any HIP call, then looked up for the stream's GPU
    if (ws_bytes(p, 1) > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_TOO_LARGE;
    int dev = 0;
    const hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                                           : hipGetDevice(&dev);
    if (e != hipSuccess || swa::noalloc_scratch(dev, &workspace) != hipSuccess) return ATTN_ERR_HIP;
    workspace_bytes = ATTN_NOALLOC_SCRATCH_BYTES;
  }
  if (workspace == nullptr || workspace_bytes < ws_bytes(p, split)) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  swa::AttnArgs a = base_args(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = static_cast<float*>(workspace);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws_array_bytes(p));
  a.kv_split = split;
  if (split > 1) a.dkv_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * ws_array_bytes(p));
  if (mask != nullptr) {
    a.mask = mask->bits;
    a.mask_words = mask->row_words;
    a.mask_ranges = mask->ranges;
  }
  if (swa::launch_bwd(p->dtype, p->head_dim, stages, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status_t attn_bwd_stages(const attn_params_t* p, int32_t stages, const void* q,
                              const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(p, nullptr, stages, q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, dq, dk, dv,
                  workspace, workspace_bytes, stream);
}

attn_status_t attn_bwd(const attn_params_t* p, const void* q, const void* k, const void* v,
                       const void* o, const float* lse, const void* dout,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* dq,
                       void* dk, void* dv, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return bwd_impl(p, nullptr, ATTN_BWD_ALL, q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, dq,
                  dk, dv, workspace, workspace_bytes, stream);
}

attn_status_t attn_bwd_noalloc(const attn_params_t* p, const void* q, const void* k, const void* v,
                               const void* o, const float* lse, const void* dout,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* dq,
                               void* dk, void* dv, void* stream) {
  return bwd_impl(p, nullptr, ATTN_BWD_ALL, q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, dq,
                  dk, dv, nullptr, 0, stream, /*use_scratch=*/true);
}

attn_status_t attn_bwd_masked(const attn_params_t* p, const attn_mask_t* mask, const void* q,
                              const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes, void* stream) {
  attn_status_t s = attn_check_params(p);
  if (s != ATTN_OK) return s;
  if (mask == nullptr) return ATTN_ERR_NULL;
  return bwd_impl(p, mask, ATTN_BWD_ALL, q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, dq, dk,
                  dv, workspace, workspace_bytes, stream);
}

const char* attn_status_str(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "inconsistent sizes";
    case ATTN_ERR_WINDOW: return "window must be >= 1";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration (head_dim, dtype, scale, or a two-sided window over sequences longer than 2^30)";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP launch error";
    case ATTN_ERR_ALIGN: return "pointer not aligned (tensors need 16 bytes)";
    case ATTN_ERR_TOO_LARGE: return "the backward's D and LSE*log2(e) exceed the no-allocation entry point's fixed scratch (ATTN_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

attn_status_t attn_tile_sizes(int32_t head_dim, int32_t dtype, int32_t* fwd_bm, int32_t* fwd_bn,
                              int32_t* bwd_bn, int32_t* bwd_bm) {
  if (!fwd_bm || !fwd_bn || !bwd_bn || !bwd_bm) return ATTN_ERR_NULL;
  int a, b, c, d;
  if (!swa::tile_sizes(dtype, head_dim, &a, &b, &c, &d)) return ATTN_ERR_UNSUPPORTED;
  *fwd_bm = a;
  *fwd_bn = b;
  *bwd_bn = c;
  *bwd_bm = d;
  return ATTN_OK;
}

static attn_status_t seq_geom(const attn_params_t* p, const int32_t* cq, const int32_t* ck, int32_t b,
                              swa::SeqGeom* g) {
  attn_status_t s = attn_check_params(p);
  if (s != ATTN_OK) return s;
  if (!cq || !ck) return ATTN_ERR_NULL;
  if (b < 0 || b >= p->batch) return ATTN_ERR_SHAPE;
  const int64_t lq = (int64_t)cq[b + 1] - cq[b], lk = (int64_t)ck[b + 1] - ck[b];
  if (lq < 0 || lk < 0) return ATTN_ERR_SHAPE;
  *g = swa::SeqGeom{lq, lk, p->window, p->causal != 0};
  return ATTN_OK;
}

attn_status_t attn_query_tile_range(const attn_params_t* p, const int32_t* cu_seqlens_q_host,
                                    const int32_t* cu_seqlens_k_host, int32_t b, int32_t qb,
                                    int32_t bm, int32_t bn, int32_t* kb_lo, int32_t* kb_hi,
                                    int32_t* full_lo, int32_t* full_hi) {
  if (!kb_lo || !kb_hi || !full_lo || !full_hi) return ATTN_ERR_NULL;
  if (bm < 1 || bn < 1 || qb < 0) return ATTN_ERR_SHAPE;
  swa::SeqGeom g;
  attn_status_t s = seq_geom(p, cu_seqlens_q_host, cu_seqlens_k_host, b, &g);
  if (s != ATTN_OK) return s;
  const swa::TileRange r = swa::query_tile_keys(g, qb, bm, bn);
  *kb_lo = r.lo;
  *kb_hi = r.hi;
  *full_lo = r.full_lo;
  *full_hi = r.full_hi;
  return ATTN_OK;
}

attn_status_t attn_key_tile_range(const attn_params_t* p, const int32_t* cu_seqlens_q_host,
                                  const int32_t* cu_seqlens_k_host, int32_t b, int32_t kb,
                                  int32_t bn, int32_t bm, int32_t* qb_lo, int32_t* qb_hi) {
  if (!qb_lo || !qb_hi) return ATTN_ERR_NULL;
  if (bm < 1 || bn < 1 || kb < 0) return ATTN_ERR_SHAPE;
  swa::SeqGeom g;
  attn_status_t s = seq_geom(p, cu_seqlens_q_host, cu_seqlens_k_host, b, &g);
  if (s != ATTN_OK) return s;
  const swa::TileRange r = swa::key_tile_queries(g, kb, bn, bm);
  *qb_lo = r.lo;
  *qb_hi = r.hi;
  return ATTN_OK;
}

// ------------------------------------------------------ linear cross-entropy

attn_status_t ce_check_params(const ce_params_t* p) {
  if (p == nullptr) return ATTN_ERR_NULL;
  if (p->n < 0 || p->vocab < 1 || p->hidden < 256 || p->hidden % 256 != 0) return ATTN_ERR_SHAPE;
  if ((int64_t)p->n * p->hidden > INT32_MAX || (int64_t)p->vocab * p->hidden > INT32_MAX) return ATTN_ERR_SHAPE;
  if (p->dtype != ATTN_BF16 && p->dtype != ATTN_F16) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

size_t ce_fwd_workspace_bytes(const ce_params_t* p) {
  if (ce_check_params(p) != ATTN_OK) return 0;
  const size_t tiles = (size_t)(p->vocab + 255) / 256;
  return round_up(tiles * (size_t)(p->n > 0 ? p->n : 1) * 8, 256);
}

static size_t ce_dz_bytes(const ce_params_t* p) {
  const size_t ldz = (size_t)(swa::ce_vocab_chunk(p->vocab) + 63) / 64 * 64;
  return round_up((size_t)(p->n > 0 ? p->n : 1) * ldz * 2, 256);
}

size_t ce_bwd_workspace_bytes(const ce_params_t* p) {
  if (ce_check_params(p) != ATTN_OK) return 0;
  size_t b = ce_dz_bytes(p);
  if (p->vocab > swa::ce_vocab_chunk(p->vocab)) b += round_up((size_t)p->n * p->hidden * 4, 256);
  return b;
}

static swa::CEArgs ce_args(const ce_params_t* p) {
  swa::CEArgs a{};
  a.n = p->n;
  a.vocab = p->vocab;
  a.hidden = p->hidden;
  return a;
}

attn_status_t ce_fwd(const ce_params_t* p, const void* h, const void* w, const int32_t* targets,
                     float* nll, float* lse, float* target_logit, void* workspace,
                     size_t workspace_bytes, void* stream) {
  attn_status_t s = ce_check_params(p);
  if (s != ATTN_OK) return s;
  const int64_t nh = (int64_t)p->n * p->hidden, vh = (int64_t)p->vocab * p->hidden;
  if ((s = check_tensor(h, nh, true)) != ATTN_OK) return s;
  if ((s = check_tensor(w, vh, true)) != ATTN_OK) return s;
  if ((s = check_tensor(targets, p->n, false)) != ATTN_OK) return s;
  if ((s = check_tensor(nll, p->n, false)) != ATTN_OK) return s;
  if ((s = check_tensor(lse, p->n, false)) != ATTN_OK) return s;
  if ((s = check_tensor(target_logit, p->n, false)) != ATTN_OK) return s;
  if (workspace == nullptr || workspace_bytes < ce_fwd_workspace_bytes(p)) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  swa::CEArgs a = ce_args(p);
  a.h = h;
  a.w = w;
  a.targets = targets;
  a.nll = nll;
  a.out_lse = lse;
  a.tgt = target_logit;
  a.part = static_cast<float*>(workspace);
  if (swa::launch_ce_fwd(p->dtype, a, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status_t ce_bwd(const ce_params_t* p, const void* h, const void* w, const int32_t* targets,
                     const float* lse, const float* dnll, void* dh, void* workspace,
                     size_t workspace_bytes, void* stream) {
  attn_status_t s = ce_check_params(p);
  if (s != ATTN_OK) return s;
  const int64_t nh = (int64_t)p->n * p->hidden, vh = (int64_t)p->vocab * p->hidden;
  if ((s = check_tensor(h, nh, true)) != ATTN_OK) return s;
  if ((s = check_tensor(w, vh, true)) != ATTN_OK) return s;
  if ((s = check_tensor(targets, p->n, false)) != ATTN_OK) return s;
  if ((s = check_tensor(lse, p->n, false)) != ATTN_OK) return s;
  if ((s = check_tensor(dnll, p->n, false)) != ATTN_OK) return s;
  if ((s = check_tensor(dh, nh, true)) != ATTN_OK) return s;
  if (workspace == nullptr || workspace_bytes < ce_bwd_workspace_bytes(p)) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  swa::CEArgs a = ce_args(p);
  a.h = h;
  a.w = w;
  a.targets = targets;
  a.lse = lse;
  a.dnll = dnll;
  a.dh = dh;
  a.dz = workspace;
  a.dh32 = reinterpret_cast<float*>(static_cast<char*>(workspace) + ce_dz_bytes(p));
  if (swa::launch_ce_bwd(p->dtype, a, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

}  // extern "C"
