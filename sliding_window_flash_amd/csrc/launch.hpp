// Internal interface between the C ABI (api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include "kernel_common.hpp"

namespace swa {

hipError_t launch_fwd(int dtype, int head_dim, const AttnArgs& a, hipStream_t st);
// stages: bit 1 = D preprocess (skipped when bit 2 is set: dQ forms D itself),
// 2 = dQ, 4 = dK/dV (run in that order)
hipError_t launch_bwd(int dtype, int head_dim, int stages, const AttnArgs& a, hipStream_t st);
bool tile_sizes(int dtype, int head_dim, int* fwd_bm, int* fwd_bn, int* bwd_bn, int* bwd_bm);
// first/last allowed blocks of a mask per 32-row and per 32-key block
// (AttnArgs::mask_ranges), written to `ranges`
hipError_t launch_mask_ranges(const AttnArgs& a, int32_t* ranges, hipStream_t st);
// dK/dV head split for small key-major grids (AttnArgs::kv_split)
int dkdv_split(int dtype, int head_dim, int heads_q, int heads_kv, int batch, int max_seqlen_k);
// Device address, on GPU `device`, of the fixed scratch array the
// no-allocation backward uses for D and LSE * log2(e) (looked up once per
// device with that device current, then cached).
hipError_t noalloc_scratch(int device, void** ptr);

}  // namespace swa
