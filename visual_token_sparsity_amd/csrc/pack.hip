// Dense packing of the selected visual KV rows (decode stage, once per
// question): SparseVILA velog summary, Sec. 3.2, decode side (the selected KV
// entries are gathered into contiguous memory so that decode reads them with
// regular, coalesced accesses) and Sec. 3.3, kernel table, decoding-attention
// row (decode attends that packed, reduced cache).
//
// A row is one token's [Hkv][D] block, a multiple of 16 bytes.  A work unit
// is 2048 16-byte vectors of destination: several whole rows when a row is
// shorter, else one slice of a row.  Each of the 256 threads issues its 8
// vector loads of K and 8 of V before the first store.  The kernel only
// streams: per selected token it reads and writes 2 x row bytes, and nothing
// else touches HBM but the index word.
#include "pack.h"

namespace sv {

namespace {

constexpr int kPackThreads = 256;
constexpr int kPackVecs = 8;                                 // per thread per matrix
constexpr int kPackUnitVecs = kPackThreads * kPackVecs;     // 16-byte vectors per unit

__global__ __launch_bounds__(kPackThreads) void pack_kernel(
    const char* __restrict__ kv, const char* __restrict__ vv, int64_t bstride_bytes,
    int64_t tstride_bytes, int N, const int32_t* __restrict__ idx, int k, int64_t nrows,
    int64_t units, int rows_per_unit, int slices_per_row, int row_vecs, char* __restrict__ kp,
    char* __restrict__ vp) {
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    // Unit u covers destination vectors [vbase, vbase + span) counted from
    // the start of row row0.
    int64_t row0;
    int vbase, span;
    if (rows_per_unit > 0) {
      row0 = u * rows_per_unit;
      const int64_t left = nrows - row0;
      span = (int)(left < rows_per_unit ? left : rows_per_unit) * row_vecs;
      vbase = 0;
    } else {
      row0 = u / slices_per_row;
      vbase = (int)(u - row0 * slices_per_row) * kPackUnitVecs;
      span = row_vecs - vbase < kPackUnitVecs ? row_vecs - vbase : kPackUnitVecs;
    }
    uint4 ka[kPackVecs], va[kPackVecs];
    int64_t dst[kPackVecs];
#pragma unroll
    for (int i = 0; i < kPackVecs; ++i) {
      const int lv = (int)threadIdx.x + i * kPackThreads;
      const int w = vbase + lv;
      const int r = w / row_vecs;
      const int v = w - r * row_vecs;
      const int64_t row = row0 + r;
      ka[i] = va[i] = make_uint4(0u, 0u, 0u, 0u);
      dst[i] = -1;
      if (lv < span) {
        dst[i] = row * (int64_t)row_vecs * 16 + (int64_t)v * 16;
        const int t = idx[row];
        if (t >= 0 && t < N) {
          const int64_t src = (row / k) * bstride_bytes + (int64_t)t * tstride_bytes + (int64_t)v * 16;
          ka[i] = *reinterpret_cast<const uint4*>(kv + src);
          va[i] = *reinterpret_cast<const uint4*>(vv + src);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kPackVecs; ++i) {
      if (dst[i] >= 0) {
        *reinterpret_cast<uint4*>(kp + dst[i]) = ka[i];
        *reinterpret_cast<uint4*>(vp + dst[i]) = va[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_pack(const void* kv, const void* vv, int64_t bstride, int64_t tstride, int N,
                       int row_elems, int elem_bytes, const int32_t* idx, int B, int k, void* kp,
                       void* vp, hipStream_t stream) {
  if (B <= 0 || k <= 0) return hipSuccess;
  const int row_vecs = row_elems * elem_bytes / 16;
  const int64_t nrows = (int64_t)B * k;
  int rows_per_unit = 0, slices_per_row = 1;
  int64_t units;
  if (row_vecs <= kPackUnitVecs) {
    rows_per_unit = kPackUnitVecs / row_vecs;
    units = (nrows + rows_per_unit - 1) / rows_per_unit;
  } else {
    slices_per_row = (row_vecs + kPackUnitVecs - 1) / kPackUnitVecs;
    units = nrows * slices_per_row;
  }
  // Enough workgroups to keep every CU streaming; a grid-stride loop covers
  // the rest.
  const int64_t cap = (int64_t)device_cu_count() * 32;
  const int grid = (int)(units < cap ? units : cap);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(kPackThreads), 0, stream, (const char*)kv,
                     (const char*)vv, bstride * elem_bytes, tstride * elem_bytes, N, idx, k, nrows,
                     units, rows_per_unit, slices_per_row, row_vecs, (char*)kp, (char*)vp);
  return hipGetLastError();
}

}  // namespace sv
