// The temperature LSE route of the sparse attention (msa_sparse_attention
// page, Parameters: return_temperature_lse, lse_temperature_scale): the
// general attention kernel also accumulates ln sum_j exp(tau * z_j) over the
// attended keys and writes it to lse_t ([total_q, Hq] fp32).
#pragma once

#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace msa {

// fmt: kFmtBf16, kFmtFp8 or kFmtE2m1 (bf16 output); tau > 0.  The plan in p
// is the general kernel's (tok_per_tile, tiles_per_req for 128-row tiles).
hipError_t launch_attention_temperature(const AttnParams& p, int fmt, float* lse_t, float tau,
                                        hipStream_t stream);

}  // namespace msa
