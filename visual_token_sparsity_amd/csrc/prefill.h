// Prefill attention of a question chunk with the retrieval fused into it
// (internal header; the entry point is sv_prefill_attend_retrieve).
#pragma once

#include "common.h"

namespace sv {

// Work plan: rows = Tq * G query rows per KV head, W waves of 32 rows per
// workgroup, RC row chunks of 32 W rows, key splits of E keys (CV visual, CT
// text), NP = Hkv * RC * W partial retrieval scores per token.
// KW > 1 (rows <= 32): one 32-row block per item and KW waves that split the
// item's keys; the CV splits of E keys run over the sequence's keys in one
// list (visual, then text), CT = 0.
struct PrefillPlan {
  int rows, W, RC, E, CV, CT, NP, KW;
};
PrefillPlan prefill_plan(int B, int Tq, int Hq, int Hkv, int N, int Tmax);
size_t prefill_part_floats(int B, int Hkv, int D, const PrefillPlan& p);

struct PrefillArgs {
  const bf16_t* q;                 // [B][Tq][Hq][D]
  const bf16_t *kv, *vv;           // visual cache, element strides vbs, vts
  const bf16_t *kt, *vt;           // text cache, element strides tbs, tts
  int64_t vbs, vts, tbs, tts;
  const int32_t* txt_len;          // [B]
  int B, Tq, Hq, Hkv, G, D, N, Tmax;
  float c2;                        // scale * log2(e)
  int rows, W, RC, E, CV, CT, NP, KW;  // the plan
  float* part;                     // split partials [B][Hkv][RC][C][32 W][D + 4]
  float* pscore;                   // partial retrieval scores [B][NP][N]
  float* out;                      // [B][Tq][Hq][D]
  float* scores;                   // [B][N] retrieval scores
  int k;                           // tokens selected per sequence (0: none)
  int32_t* idx;                    // [B][k]
  uint32_t* ctl;                   // [2B] completion counters (stride kCtrStride), zero between calls
  void* long_ws;                   // rows of more than 2048 tokens: the parallel select's
                                   // workspace (prefill_long_select_bytes), else null
};

// Workspace of the parallel select of rows of more than 2048 tokens (0 for
// shorter rows); zero between calls.
size_t prefill_long_select_bytes(int B, int N);

// Attention + combine, retrieval scores into `scores` [B][N], then (k > 0)
// the top-k per sequence into idx [B][k].
hipError_t launch_prefill(const PrefillArgs& a, float* scores, int k, int32_t* idx,
                          hipStream_t stream);

}  // namespace sv
