// Dense packing of the selected visual KV rows (internal header).
#pragma once

#include "common.h"

namespace sv {

// kp/vp[b*k + j] = kv/vv row idx[b*k + j] of sequence b (a zero row for an
// index outside [0, N)).  Strides in elements; rows of row_elems elements,
// row_elems * elem_bytes a multiple of 16.
hipError_t launch_pack(const void* kv, const void* vv, int64_t bstride, int64_t tstride, int N,
                       int row_elems, int elem_bytes, const int32_t* idx, int B, int k, void* kp,
                       void* vp, hipStream_t stream);

}  // namespace sv
