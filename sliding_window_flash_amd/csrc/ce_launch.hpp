// Internal interface between the C ABI (api.hip) and the cross-entropy
// kernels (ce_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

struct CEArgs {
  const void* h;           // hidden states [n, hidden]
  const void* w;           // head [vocab, hidden]
  const int32_t* targets;  // [n]
  const float* lse;        // [n] natural log (backward input)
  const float* dnll;       // [n] upstream gradient (backward input)
  float* nll;              // [n] (forward outputs)
  float* out_lse;          // [n]
  float* tgt;              // [n]
  float* part;             // forward workspace: [ceil(vocab / 256)][n] (max*log2 e, sum)
  void* dz;                // backward workspace: one chunk of dz, [n, vc]
  float* dh32;             // backward workspace: fp32 dH accumulator [n, hidden]
  void* dh;                // backward output [n, hidden]
  int32_t n, vocab, hidden;
  int32_t v0, vc;          // backward: the chunk [v0, v0 + vc) of the vocabulary
  int32_t ldz;             // backward: dz row stride, vc rounded up to 64 (padding columns hold 0)
};

hipError_t launch_ce_fwd(int dtype, const CEArgs& a, hipStream_t st);
hipError_t launch_ce_bwd(int dtype, const CEArgs& a, hipStream_t st);
int ce_vocab_chunk(int vocab);  // vocabulary entries per backward chunk

}  // namespace swa
