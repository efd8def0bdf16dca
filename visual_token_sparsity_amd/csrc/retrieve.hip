// Query-aware retrieval for the decode stage: relevance scan + exact top-k in
// one kernel (SparseVILA velog summary, Sec. 3.2, Query-Aware Token
// Selection; xllm-io review, core formulas: TopK(Query . KV_Cache, k)).
//
// Workgroup (i, b) runs scan item i of sequence b (decode_items.h).  With
// k > 0 every item publishes its scores with device-coherent stores and bumps
// a per-sequence counter; the last item of a sequence runs the exact top-k of
// the whole score row and resets the counter, so the workspace is ready for
// the next call.  Also: the top-k of independent rows (per-frame pruning).
#include "decode_items.h"

namespace sv {

template <typename T>
__global__ __launch_bounds__(kItemThreads) void scan_select_kernel(ScanArgs a) {
  extern __shared__ __align__(16) char smem[];
  int q_of = -1;
  const int b = blockIdx.y;
  if (scan_item<T, short_scan_cpl<T>()>(a, b, blockIdx.x, smem, q_of)) select_item(a, b, smem, q_of);
}

int scan_rows_per_item(int B, int N, int LPR, int nseg) {
  // About 1024 items in all (B of them per row slice when each item scans one
  // sequence), each wave with a short run of rows (whole rows per wave when a
  // row has several segments).
  return scan_rows_for_items(B, N, LPR, nseg, 1024);
}

int scan_rows_for_items(int B, int N, int LPR, int nseg, long target_items) {
  if (target_items < 1) target_items = 1;
  long per_seq = (target_items + B - 1) / B;
  const int rps = kWave / LPR;
  const long min_rows = (long)kItemWaves * (nseg > 1 ? 1 : rps);
  long rows = (N + per_seq - 1) / per_seq;
  if (rows < min_rows) rows = min_rows;
  rows = ((rows + min_rows - 1) / min_rows) * min_rows;
  return (int)rows;
}

hipError_t launch_retrieve(const void* q, int B, int Tq, int Hq, const void* kv, int64_t bstride,
                           int64_t tstride, int N, int Hkv, int D, int dtype, float* scores, int k,
                           int32_t* idx_out, uint32_t* counters, int rows_per_item,
                           hipStream_t stream) {
  const int VE = dtype == 1 ? 8 : 4;
  ScanArgs a{};
  a.q = q;
  a.Tq = Tq;
  a.Hq = Hq;
  a.G = Hq / Hkv;
  a.kv = kv;
  a.bstride = bstride;
  a.tstride = tstride;
  a.N = N;
  a.D = D;
  a.C = Hkv * D / VE;
  // The fused kernel's short-row unit size: both paths sum in the same order.
  scan_geometry(a.C, &a.nseg, &a.LPR, short_scan_cpl(dtype));
  a.rows_per_item = rows_per_item > 0 ? rows_per_item : scan_rows_per_item(B, N, a.LPR, a.nseg);
  a.items_per_seq = (N + a.rows_per_item - 1) / a.rows_per_item;
  a.scores = scores;
  a.k = k;
  a.idx = idx_out;
  a.seq_ctr = counters;
  a.ready = nullptr;
  const size_t lds = scan_smem_bytes(a.nseg, a.LPR, VE, false, short_scan_cpl(dtype));
  const dim3 grid(a.items_per_seq, B);
  if (dtype == 1)
    hipLaunchKernelGGL(scan_select_kernel<bf16_t>, grid, dim3(kItemThreads), lds, stream, a);
  else
    hipLaunchKernelGGL(scan_select_kernel<float>, grid, dim3(kItemThreads), lds, stream, a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Top-k of independent rows, one workgroup per row (used for per-frame pruning)
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kItemThreads) void topk_rows_kernel(const float* __restrict__ vals,
                                                               int64_t row_stride, int N, int k,
                                                               int32_t* __restrict__ out) {
  __shared__ SelectSmem<kItemWaves> sm;
  if (k <= 0) return;
  const float* row = vals + (int64_t)blockIdx.x * row_stride;
  if (N <= kItemThreads * kSelKpt) {
    block_topk<kItemWaves, kSelKpt, false, true>(row, N, k, out + (int64_t)blockIdx.x * k, sm);
  } else {
    block_topk<kItemWaves, kSelKpt, false, false>(row, N, k, out + (int64_t)blockIdx.x * k, sm);
  }
}

hipError_t launch_topk_rows(const float* vals, int rows, int64_t row_stride, int N, int k,
                            int32_t* out, hipStream_t stream) {
  if (k <= 0 || rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_rows_kernel, dim3(rows), dim3(kItemThreads), 0, stream, vals,
                     row_stride, N, k, out);
  return hipGetLastError();
}

}  // namespace sv
