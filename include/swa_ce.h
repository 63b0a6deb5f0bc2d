/*
 * Linear cross-entropy without the logits tensor: C ABI for MI355X (gfx950).
 *
 * The mlx-train-perf README, the passage on its logit-free linear
 * cross-entropy: the loss and its gradient are computed without building the
 * (N, V) logits; the forward regenerates logits tile by tile over the
 * vocabulary and returns three N-length arrays (the per-token loss, the
 * log-sum-exp and the target logit); the backward recomputes the tiles it
 * needs and returns the gradient back into the hidden states.
 *
 * For hidden states H [n, hidden], head W [vocab, hidden] (row-major, the
 * I/O dtype) and targets y [n] (int32, in [0, vocab)):
 *   z = H W^T (never stored), lse_i = log sum_v exp(z_iv),
 *   target_i = z_{i, y_i}, nll_i = lse_i - target_i (fp32 outputs);
 *   backward, for an upstream gradient g = dL/dnll [n] (fp32):
 *   dH_i = g_i (sum_v softmax(z_i)_v W_v - W_{y_i})   (the I/O dtype).
 * The head gets no gradient (it is not trained).
 *
 * Status codes and dtypes are those of swa_attn.h. All pointers are device
 * memory owned by the caller; nothing is allocated, nothing synchronises.
 */
#ifndef SWA_CE_H
#define SWA_CE_H

#include "swa_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t n;      /* tokens, >= 0 */
  int32_t vocab;  /* V >= 1 */
  int32_t hidden; /* a multiple of 256, >= 256 */
  int32_t dtype;  /* ATTN_BF16 or ATTN_F16 (ATTN_F32 is refused: ATTN_ERR_UNSUPPORTED) */
} ce_params_t;

/* Validate parameters without launching anything: ATTN_ERR_NULL (p NULL),
 * ATTN_ERR_SHAPE (n < 0, vocab < 1, hidden not a positive multiple of 256,
 * n * hidden or vocab * hidden >= 2^31), ATTN_ERR_UNSUPPORTED (dtype). */
attn_status_t ce_check_params(const ce_params_t* p);

/* Forward workspace: per (256-word vocabulary tile, token) partial maxima and
 * sums, 8 bytes each, 256-byte aligned. 0 if the parameters are invalid. */
size_t ce_fwd_workspace_bytes(const ce_params_t* p);

/* Forward: writes nll, lse (natural log) and target_logit, fp32 [n] each. A
 * target outside [0, vocab) yields NaN target_logit and nll for that token.
 * h, w: 16-byte aligned; targets and the outputs 4-byte aligned; the
 * workspace (ce_fwd_workspace_bytes) 16-byte aligned, contents ignored.
 * Errors: the checks above, ATTN_ERR_NULL / ATTN_ERR_ALIGN for pointers,
 * ATTN_ERR_WORKSPACE, ATTN_ERR_HIP at launch. */
attn_status_t ce_fwd(const ce_params_t* p, const void* h, const void* w, const int32_t* targets,
                     float* nll, float* lse, float* target_logit, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Backward workspace: one vocabulary chunk of dz = dL/dz in the I/O dtype
 * (n x at most 16,384 columns) and, when the vocabulary spans several chunks,
 * an fp32 dH accumulator [n, hidden]. 0 if the parameters are invalid. */
size_t ce_bwd_workspace_bytes(const ce_params_t* p);

/* Backward: writes dh [n, hidden] (I/O dtype) from h, w, targets, the
 * forward's lse and dnll (fp32 [n]). Same alignment and error rules as
 * ce_fwd (dh 16-byte aligned). */
attn_status_t ce_bwd(const ce_params_t* p, const void* h, const void* w, const int32_t* targets,
                     const float* lse, const float* dnll, void* dh, void* workspace,
                     size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_CE_H */
