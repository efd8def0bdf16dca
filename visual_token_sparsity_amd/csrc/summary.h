// Summary-token salience (internal header).
#pragma once

#include "common.h"

namespace sv {

// Largest supported sizes: summary tokens, tokens per frame, and S*N logits
// held in LDS by one workgroup.
constexpr int kSummaryMaxS = 16;
constexpr int kSummaryMaxN = 4096;
constexpr int kSummaryMaxLogits = 12288;

// sal[f][j] = (1/H) sum_h (1/S) sum_{s<S} softmax_j(scale * q[f,h,s,:] . k[f,h,j,:]),
// q and k [F][H][N][D] bf16; colh_ws holds F*H*N floats.  Then, if keep > 0,
// the keep largest sal[f][.] per frame into idx_out [F][keep] (ascending).
hipError_t launch_summary_salience(const void* q, const void* k, int F, int H, int N, int D, int S,
                                   float scale, int keep, float* colh_ws, float* sal,
                                   int32_t* idx_out, hipStream_t stream);

}  // namespace sv
