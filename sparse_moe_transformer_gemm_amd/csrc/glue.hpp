// Launch of the stack glue kernel (norm.hip): the block's combine folded into
// the residual add and the next block's pre-norm.
#pragma once

#include "common.hpp"

namespace moe {

// The combine, then resid_out = bf16(resid + m) and, with gain, nout = RMSNorm
// of it: the bytes of launch_combine, launch_residual_add and launch_rmsnorm in
// one pass (mout, if not null, receives m).
hipError_t launch_combine_residual_rmsnorm(const float* y_sorted, const int32_t* pair_row,
                                           const float* topk_w, const uint16_t* resid,
                                           const uint16_t* gain, int T, int d, int k, float eps,
                                           uint16_t* mout, uint16_t* resid_out, uint16_t* nout,
                                           hipStream_t stream);

}  // namespace moe
