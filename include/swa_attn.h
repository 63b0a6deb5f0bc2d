/*
 * swa_attn.h - C ABI of the sliding-window flash-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (the pages it follows are cited by title and
 * section):
 *
 *   Tiled, memory-linear scaled-dot-product attention, forward and backward,
 *   with causal and sliding-window masks, grouped-query heads and ragged packed
 *   batches. The forward saves only O and the per-row log-sum-exp; the backward
 *   recomputes score tiles from them and from D = rowsum(dO * O), and never
 *   holds the full score matrix ("Off NVIDIA, you fix the platform yourself",
 *   sections "What was broken?" and "What did fixing it take?"; the
 *   mlx-train-perf README, flash-attention passage: O(N) saved state, the
 *   output and the log-sum-exp, tiles recomputed in the backward).
 *
 *   Visibility. Sequence b has L_q query and L_k key tokens; query i sits at
 *   key position p = i + L_k - L_q (the queries are the last positions). Key j
 *   is visible to query i iff j <= p and p - j < window (causal), or iff
 *   |p - j| < window (non-causal: a two-sided window; any window >=
 *   max(L_q, L_k) is full attention). window = 1 sees only the token itself
 *   (the lab record's gradient-parity sweep runs windows causal and not).
 *   With L_q > L_k the first L_q - L_k positions are negative: under the
 *   causal mask those queries see no key. A query that sees no key gets
 *   O = 0, LSE = -inf and dQ = 0, and adds nothing to dK and dV.
 *   Key tiles lying wholly outside a query tile's window are skipped; cells on
 *   the window edge are masked ("What did fixing it take?": skip blocks
 *   entirely outside the window, mask the cells at its edge). A query tile's
 *   first visited key tile need not be tile zero, and key tiles that no query
 *   sees get exact-zero dK and dV (same section: the two assumptions that
 *   broke silently).
 *
 * Layouts (all row-major, contiguous, device memory, 16-byte aligned):
 *   Q, O, dO, dQ : [total_q, heads_q, head_dim]
 *   K, V, dK, dV : [total_k, heads_kv, head_dim]
 *   LSE          : [heads_q, total_q] fp32, natural log of the scaled scores
 *   cu_seqlens_q : [batch + 1] int32, cu_seqlens_q[0] = 0, last = total_q
 *   cu_seqlens_k : [batch + 1] int32, likewise with total_k
 *   Head h of Q uses KV head h / (heads_q / heads_kv) (contiguous groups).
 *
 * Ownership: the caller owns every buffer, including the backward workspace.
 * The library allocates no device memory and keeps no state between calls
 * (except attn_bwd_noalloc's fixed per-GPU array, described there), so all
 * device memory is visible to the caller's allocator. Every element of
 * every output is written (zeros where the definition gives zero): outputs
 * need no clearing.
 *
 * Execution: calls enqueue kernels on `stream` (a hipStream_t; NULL = the
 * default stream) and return. They never synchronise, copy between host and
 * device or read device memory on the host. They are reentrant.
 *
 * Errors: every argument check happens before any launch and returns a status
 * code; nothing is launched on error. Unsupported inputs are refused up front,
 * never silently routed elsewhere (the mlx-train-perf README's refusal table:
 * unsupported configurations raise at enable time rather than fail mid-run;
 * "auto" never silently downgrades). There is no fallback path and no
 * exception crosses this boundary.
 *
 * Preconditions the host cannot check without reading device memory:
 * cu_seqlens are non-decreasing, and every sequence has L_q <= max_seqlen_q
 * and L_k <= max_seqlen_k.
 */
#ifndef SWA_ATTN_H
#define SWA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_F32 = 0,  /* Q, K, V, O, dO, dQ, dK, dV are float32 */
  ATTN_BF16 = 1, /* ... are bfloat16; accumulation and score tiles stay fp32 */
  ATTN_F16 = 2   /* ... are IEEE half; accumulation and score tiles stay fp32 */
} attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* sizes inconsistent (batch < 1, heads_q % heads_kv, heads_q > 16384 or
                               128 x heads_q x head_dim x element bytes >= 2^31, totals, more than
                               2^31 - 1 work items: ceil(max_seqlen / 32) x heads x batch ...) */
  ATTN_ERR_WINDOW = 3,      /* window < 1 */
  ATTN_ERR_UNSUPPORTED = 4, /* head_dim not 64/128 (256, 512: 16-bit dtypes only), unknown dtype, scale <= 0,
                               a two-sided window below max(max_seqlen_q, max_seqlen_k) when that
                               maximum exceeds 2^30 */
  ATTN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than attn_bwd_workspace_bytes */
  ATTN_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
  ATTN_ERR_ALIGN = 7,       /* a tensor pointer is not 16-byte aligned */
  ATTN_ERR_TOO_LARGE = 8    /* attn_bwd_noalloc: the problem needs more than ATTN_NOALLOC_SCRATCH_BYTES */
} attn_status_t;

typedef struct {
  int32_t batch;        /* B >= 1 packed sequences */
  int32_t heads_q;      /* query heads, a multiple of heads_kv */
  int32_t heads_kv;     /* key/value heads; G = heads_q / heads_kv queries share one */
  int32_t head_dim;     /* 64 or 128; 256 and 512 for bf16 and fp16 */
  int32_t total_q;      /* cu_seqlens_q[B] */
  int32_t total_k;      /* cu_seqlens_k[B] */
  int32_t max_seqlen_q; /* >= every L_q; sizes the launch grid (no device reads) */
  int32_t max_seqlen_k; /* >= every L_k */
  int32_t window;       /* >= 1; INT32_MAX (or any value >= max(max_seqlen_q, max_seqlen_k)) is no window */
  int32_t causal;       /* 1 causal; 0 two-sided window (full attention if window >= max(L_q, L_k)) */
  float scale;          /* softmax scale, finite and > 0, e.g. 1/sqrt(head_dim) */
  int32_t dtype;        /* attn_dtype_t */
} attn_params_t;

/* Forward. Writes O [total_q, heads_q, head_dim] (dtype) and LSE [heads_q,
 * total_q] (fp32). */
attn_status_t attn_fwd(const attn_params_t* p, const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* o,
                       float* lse, void* stream);

/* Bytes of device workspace attn_bwd needs for these parameters: -D =
 * -rowsum(dO * O) and LSE * log2(e), each fp32 [heads_q, total_q] and 256-byte
 * aligned; plus, when the key tiles (128 keys) x heads_kv x batch are fewer
 * than the GPU's 256 compute units, fp32 partial dK and dV [parts][2][total_k,
 * heads_kv, head_dim] for the dK/dV launch, which then splits each KV group's
 * query heads over 2, 4, ... workgroups (bf16 and fp16 at head_dim 64 and 128)
 * and adds the parts in a second launch. 0 if the parameters are invalid. */
size_t attn_bwd_workspace_bytes(const attn_params_t* p);

/* Backward: the vector-Jacobian product of sum(O * dO). Reads Q, K, V, O, LSE
 * (as written by attn_fwd with the same parameters) and dO; writes dQ, dK, dV
 * (dtype) in full. `workspace` must hold attn_bwd_workspace_bytes(p) bytes;
 * its contents on entry do not matter. */
attn_status_t attn_bwd(const attn_params_t* p, const void* q, const void* k, const void* v,
                       const void* o, const float* lse, const void* dout,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* dq,
                       void* dk, void* dv, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Bytes of the fixed device array attn_bwd_noalloc keeps per GPU. */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid hipMalloc). The backward's D and LSE * log2(e) go to a fixed
 * array of ATTN_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on, from the first call there until the process ends. The call
 * allocates nothing; the first call on a GPU looks up the array's device
 * address (the HIP runtime may load the library's code object on that GPU
 * then), later calls reuse it. Same arguments (minus the workspace), outputs
 * and errors as attn_bwd, plus ATTN_ERR_TOO_LARGE, returned before any HIP
 * call, when attn_bwd_workspace_bytes(p) exceeds ATTN_NOALLOC_SCRATCH_BYTES
 * (heads_q x total_q above about 4.19 million rows). The GPU is the one of
 * `stream` (the current device for NULL).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that can overlap in time on one GPU (other streams, other
 * host threads) race and give wrong results; calls ordered on one stream are
 * safe. Nothing in it needs clearing first: the dQ launch writes every entry
 * the dK/dV launch reads. */
attn_status_t attn_bwd_noalloc(const attn_params_t* p, const void* q, const void* k, const void* v,
                               const void* o, const float* lse, const void* dout,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* dq,
                               void* dk, void* dv, void* stream);

/* The backward's stages, for callers that schedule them themselves:
 *   ATTN_BWD_DELTA: -D = -rowsum(dO * O) and LSE * log2(e) into the workspace;
 *   ATTN_BWD_DQ:    dQ (reads Q, K, V, O, LSE and dO); it forms D and
 *                   LSE * log2(e) for its rows itself and writes them into the
 *                   workspace as DELTA does, so a call that selects both runs
 *                   only DQ;
 *   ATTN_BWD_DKDV:  dK and dV (reads Q, K, V, dO and the workspace).
 * DKDV needs a completed DELTA or DQ of the same call parameters and
 * workspace. attn_bwd is attn_bwd_stages with all of them: DQ, then DKDV, on
 * one stream. Same arguments and checks as attn_bwd; pointers a selected
 * stage does not read or write may be NULL (O and LSE are read only by DELTA
 * and DQ, dQ written only by DQ, dK and dV only by DKDV). */
typedef enum {
  ATTN_BWD_DELTA = 1,
  ATTN_BWD_DQ = 2,
  ATTN_BWD_DKDV = 4,
  ATTN_BWD_ALL = 7
} attn_bwd_stage_t;

attn_status_t attn_bwd_stages(const attn_params_t* p, int32_t stages, const void* q,
                              const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes, void* stream);

/* An arbitrary boolean mask combined with the window.
 *
 * "Off NVIDIA, you fix the platform yourself" (labs.layer2c.com), list of
 * what is not proved: a window combined with an arbitrary mask still falls
 * back to the full score matrix in training; its backward-memory record entry
 * measures against the boolean mask mlx-lm passes. Here such a mask is one
 * boolean matrix per packed batch, shared by every head: cell (i, j) of
 * sequence b is visible iff the window shows it (attn_params_t) AND the mask
 * allows it. The kernels still visit only the window's tiles, so time and
 * memory stay linear in the sequence length; the mask adds one bit per
 * (query token, key) of input.
 *
 * Layout: row t (packed query token t = cu_seqlens_q[b] + i) is `row_words`
 * consecutive uint32 words; bit (j % 32) of word (j / 32) allows key j of that
 * token's sequence (0-based within the sequence, i.e. packed key
 * cu_seqlens_k[b] + j). Bits for j >= L_k are ignored. A query whose visible
 * set is empty gets O = 0, LSE = -inf and contributes no gradient.
 * Ownership: device memory owned by the caller, only read. */
typedef struct {
  const uint32_t* bits; /* device, [total_q, row_words], 16-byte aligned */
  int64_t row_words;    /* a multiple of 4, >= ceil(max_seqlen_k / 32), < 2^24 */
  const int32_t* ranges; /* optional (NULL: none): device, what attn_mask_ranges wrote for this
                            mask, these cu_seqlens and these parameters; 4-byte aligned */
} attn_mask_t;

/* Bytes of the `ranges` buffer attn_mask_ranges fills for these parameters:
 * 2 x batch x (ceil(max_seqlen_q / 32) + ceil(max_seqlen_k / 32)) int32. 0 if
 * the parameters are invalid. */
size_t attn_mask_ranges_bytes(const attn_params_t* p);

/* Where the mask's allowed bits lie, so that the masked calls skip the tiles
 * the mask empties (the lab's list of what is not proved: a window combined
 * with an arbitrary mask still falls back to the full score matrix; here the
 * window's tiles are visited as without a mask, and with these ranges only
 * those that hold an allowed bit). For each sequence and 32-row block of its
 * queries, the first and last 32-key block in which some row of the block
 * allows a key the window can show it; for each 32-key block, the first and
 * last 32-row block in which some row the window lets see it allows one of
 * its keys ((1, 0) when none). One launch on `stream`, reading the mask words
 * inside the window's band only. The kernels narrow each query tile's key
 * range and each key tile's query range to these; a tile outside them has
 * every cell masked and would add nothing, so outputs are the same as without
 * ranges. Compute once per mask and reuse it across calls (layers) that share
 * the mask and the parameters. Same checks as attn_fwd_masked, plus
 * ATTN_ERR_NULL / ATTN_ERR_ALIGN for `ranges`. */
attn_status_t attn_mask_ranges(const attn_params_t* p, const attn_mask_t* mask, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, int32_t* ranges, void* stream);

/* attn_fwd with a mask. Same outputs and errors as attn_fwd; also
 * ATTN_ERR_NULL if `mask` or (total_q > 0) `mask->bits` is NULL, ATTN_ERR_ALIGN
 * if `bits` is not 16-byte aligned, ATTN_ERR_SHAPE if `row_words` is not a
 * multiple of 4 or is below ceil(max_seqlen_k / 32), ATTN_ERR_UNSUPPORTED if it
 * is 2^24 or more (a 64-row tile of the mask must span fewer than 2^32 bytes). */
attn_status_t attn_fwd_masked(const attn_params_t* p, const attn_mask_t* mask, const void* q,
                              const void* k, const void* v, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, void* o, float* lse, void* stream);

/* attn_bwd with a mask (the one the forward used). Same outputs, workspace
 * and errors as attn_bwd, plus the mask checks of attn_fwd_masked. */
attn_status_t attn_bwd_masked(const attn_params_t* p, const attn_mask_t* mask, const void* q,
                              const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* attn_status_str(attn_status_t s);

/* Validate parameters without launching anything (the same checks attn_fwd and
 * attn_bwd make first). Pointers are not inspected. */
attn_status_t attn_check_params(const attn_params_t* p);

/* Tile sizes the compiled kernels use for (head_dim, dtype): query rows per
 * forward/dQ workgroup counted over its heads (4 waves of 32 rows: with a KV
 * group of 4k query heads a workgroup takes 4 heads x 32 rows, with 2k heads
 * 2 x 64, otherwise 1 x 128), key rows per forward/dQ step, key rows per dK/dV
 * tile and query rows per dK/dV step. Returns ATTN_ERR_UNSUPPORTED for an
 * unsupported pair. Host only. */
attn_status_t attn_tile_sizes(int32_t head_dim, int32_t dtype, int32_t* fwd_bm,
                              int32_t* fwd_bn, int32_t* bwd_bn, int32_t* bwd_bm);

/* Block-range scheduler, host build (the kernels run the same code). For query
 * tile qb of sequence b (tile = rows [qb*bm, qb*bm+bm)), the range of key tiles
 * of size bn the kernels visit: [*kb_lo, *kb_hi] (empty when *kb_lo > *kb_hi),
 * and the sub-range [*full_lo, *full_hi] of tiles in which every cell is visible
 * (no per-cell mask needed; empty when *full_lo > *full_hi). cu_seqlens_q/k are
 * HOST arrays here. */
attn_status_t attn_query_tile_range(const attn_params_t* p, const int32_t* cu_seqlens_q_host,
                                    const int32_t* cu_seqlens_k_host, int32_t b, int32_t qb,
                                    int32_t bm, int32_t bn, int32_t* kb_lo, int32_t* kb_hi,
                                    int32_t* full_lo, int32_t* full_hi);

/* Key-major counterpart used by the dK/dV kernel: for key tile kb of sequence
 * b (size bn), the query tiles of size bm that see it: [*qb_lo, *qb_hi], empty
 * when *qb_lo > *qb_hi (then dK and dV of that tile are written as zeros). */
attn_status_t attn_key_tile_range(const attn_params_t* p, const int32_t* cu_seqlens_q_host,
                                  const int32_t* cu_seqlens_k_host, int32_t b, int32_t kb,
                                  int32_t bn, int32_t bm, int32_t* qb_lo, int32_t* qb_hi);

#ifdef __cplusplus
}
#endif

#endif /* SWA_ATTN_H */
