// Query-aware retrieval for the decode stage: relevance scan + exact top-k,
// in one kernel.
//
// SparseVILA velog summary, Sec. 3.2 (Query-Aware Token Selection): the
// current query scores every cached vision token and only the top-k are
// activated.  xllm-io review, core formulas: TopK(Query . KV_Cache, k).
//
// Scan.  s[b,t] = sum_g qhat[b,g,:] . K[b,t,g,:] where qhat[b,g] is the sum of
// the query over the Tq query tokens and the G query heads sharing KV head g.
// The sum is linear, so summing the queries first gives the same score as
// summing per-head logits.  Decode is HBM-bound: every retained key row is
// read exactly once as contiguous 16-byte vectors.  A lane group of LPR lanes
// covers one token row (Hkv*D elements); each wave walks a contiguous run of
// rows with the next rows' loads already in flight, and the key loads of the
// first rows are issued before the query is summed.
//
// Select.  Every workgroup of sequence b publishes its scores with
// device-coherent stores, waits for them to complete and bumps a counter; the
// last one runs the exact top-k of the whole score row (select.h, reading
// with device-coherent loads) and resets the counter to zero, so the
// workspace is ready for the next call.
#include "common.h"
#include "select.h"

namespace sv {

constexpr int kScanWaves = 4;
constexpr int kSelKpt = 8;  // keys per thread kept in registers by the select

template <typename T, int CPL, int LPR>
__global__ __launch_bounds__(kScanWaves* kWave) void retrieve_kernel(
    const T* __restrict__ q, int Tq, int Hq, int G, const T* __restrict__ kv, int64_t bstride,
    int64_t tstride, int N, int D, int rows_per_wave, float* __restrict__ scores, int k,
    int32_t* __restrict__ idx_out, uint32_t* __restrict__ counters) {
  constexpr int VE = Vec<T>::kElems;
  constexpr int RPW = kWave / LPR;  // rows per wave per step
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int b = blockIdx.y;
  const int sub = lane % LPR;
  const int rsub = lane / LPR;

  const T* base = kv + (int64_t)b * bstride;
  float* srow = scores + (int64_t)b * N;
  const int r_begin = (blockIdx.x * kScanWaves + wave) * rows_per_wave;
  int r_end = r_begin + rows_per_wave;
  r_end = r_end < N ? r_end : N;

  // First rows' keys in flight before anything else.
  Vec<T> nxt[CPL];
  {
    const int r = r_begin + rsub;
    if (r < r_end) {
      const T* row = base + (int64_t)r * tstride;
#pragma unroll
      for (int j = 0; j < CPL; ++j) nxt[j].load_stream(row + (sub + j * LPR) * VE);
    } else {
#pragma unroll
      for (int j = 0; j < CPL; ++j) nxt[j].zero();
    }
  }

  // qhat for this lane's chunks: chunk j covers row elements [(sub + j*LPR)*VE, +VE).
  float qh[CPL][VE];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int e0 = (sub + j * LPR) * VE;
    const int g = e0 / D, d0 = e0 % D;
#pragma unroll
    for (int v = 0; v < VE; ++v) qh[j][v] = 0.f;
    for (int tau = 0; tau < Tq; ++tau) {
      for (int i = 0; i < G; ++i) {
        Vec<T> x;
        x.load(q + ((int64_t)(b * Tq + tau) * Hq + g * G + i) * D + d0);
        float f[VE];
        x.to_f32(f);
#pragma unroll
        for (int v = 0; v < VE; ++v) qh[j][v] += f[v];
      }
    }
  }

  for (int r0 = r_begin; r0 < r_end; r0 += RPW) {
    Vec<T> cur[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) cur[j] = nxt[j];
    // Prefetch the next step's rows.
    {
      const int r = r0 + RPW + rsub;
      if (r < r_end) {
        const T* row = base + (int64_t)r * tstride;
#pragma unroll
        for (int j = 0; j < CPL; ++j) nxt[j].load_stream(row + (sub + j * LPR) * VE);
      }
    }
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float f[VE];
      cur[j].to_f32(f);
#pragma unroll
      for (int v = 0; v < VE; ++v) acc = fmaf(qh[j][v], f[v], acc);
    }
    acc = group_sum<LPR>(acc);
    const int r = r0 + rsub;
    if (r < r_end && sub == 0) {
      if (k > 0)
        store_shared_dev(srow + r, acc);  // read back by the selecting workgroup
      else
        srow[r] = acc;
    }
  }

  if (k <= 0) return;
  __shared__ SelectSmem<kScanWaves> sm;
  __shared__ uint32_t s_last;
  wait_stores_complete();
  __syncthreads();
  if (threadIdx.x == 0) s_last = counter_add(&counters[b], 1u) == gridDim.x - 1 ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  block_topk<kScanWaves, kSelKpt, true>(srow, N, k, idx_out + (int64_t)b * k, sm);
  if (threadIdx.x == 0) counter_reset(&counters[b]);
}

template <typename T, int CPL, int LPR>
static hipError_t retrieve_go(const void* q, int B, int Tq, int Hq, int G, const void* kv,
                              int64_t bs, int64_t ts, int N, int D, float* scores, int k,
                              int32_t* idx, uint32_t* counters, hipStream_t st) {
  constexpr int RPW = kWave / LPR;
  // About 16 resident waves per CU on 256 CUs; each wave walks a run of rows.
  const long target_waves = 4096;
  long waves_per_seq = (target_waves + B - 1) / B;
  const long max_waves = (N + RPW - 1) / RPW;
  if (waves_per_seq > max_waves) waves_per_seq = max_waves;
  int rows_per_wave = (int)((N + waves_per_seq - 1) / waves_per_seq);
  rows_per_wave = ((rows_per_wave + RPW - 1) / RPW) * RPW;
  const int waves = (N + rows_per_wave - 1) / rows_per_wave;
  const int blocks = (waves + kScanWaves - 1) / kScanWaves;
  hipLaunchKernelGGL((retrieve_kernel<T, CPL, LPR>), dim3(blocks, B), dim3(kScanWaves * kWave), 0,
                     st, (const T*)q, Tq, Hq, G, (const T*)kv, bs, ts, N, D, rows_per_wave,
                     scores, k, idx, counters);
  return hipGetLastError();
}

template <typename T>
static hipError_t retrieve_dispatch(const void* q, int B, int Tq, int Hq, int G, const void* kv,
                                    int64_t bs, int64_t ts, int N, int R, int D, float* scores,
                                    int k, int32_t* idx, uint32_t* ctr, hipStream_t st) {
  constexpr int VE = Vec<T>::kElems;
  const int C = R / VE;  // 16-byte chunks per token row
  // Each lane keeps CPL chunks of qhat; a row is covered by LPR = C / CPL lanes.
  switch (C) {
    case 8: return retrieve_go<T, 8, 1>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, k, idx, ctr, st);
    case 16: return retrieve_go<T, 8, 2>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, k, idx, ctr, st);
    case 32: return retrieve_go<T, 8, 4>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, k, idx, ctr, st);
    case 64: return retrieve_go<T, 8, 8>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, k, idx, ctr, st);
    case 128: return retrieve_go<T, 8, 16>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, k, idx, ctr, st);
    case 256: return retrieve_go<T, 8, 32>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, k, idx, ctr, st);
    case 512: return retrieve_go<T, 8, 64>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, k, idx, ctr, st);
    case 1024: return retrieve_go<T, 16, 64>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, k, idx, ctr, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_retrieve(const void* q, int B, int Tq, int Hq, const void* kv, int64_t bstride,
                           int64_t tstride, int N, int Hkv, int D, int dtype, float* scores, int k,
                           int32_t* idx_out, uint32_t* counters, hipStream_t stream) {
  const int G = Hq / Hkv;
  const int R = Hkv * D;
  if (dtype == 1)
    return retrieve_dispatch<bf16_t>(q, B, Tq, Hq, G, kv, bstride, tstride, N, R, D, scores, k,
                                     idx_out, counters, stream);
  return retrieve_dispatch<float>(q, B, Tq, Hq, G, kv, bstride, tstride, N, R, D, scores, k,
                                  idx_out, counters, stream);
}

// ----------------------------------------------------------------------------
// Top-k of independent rows, one workgroup per row (used for per-frame pruning)
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kScanWaves* kWave) void topk_rows_kernel(const float* __restrict__ vals,
                                                                    int64_t row_stride, int N,
                                                                    int k, int32_t* __restrict__ out) {
  __shared__ SelectSmem<kScanWaves> sm;
  if (k <= 0) return;
  block_topk<kScanWaves, kSelKpt, false>(vals + (int64_t)blockIdx.x * row_stride, N, k,
                                  out + (int64_t)blockIdx.x * k, sm);
}

hipError_t launch_topk_rows(const float* vals, int rows, int64_t row_stride, int N, int k,
                            int32_t* out, hipStream_t stream) {
  if (k <= 0 || rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_rows_kernel, dim3(rows), dim3(kScanWaves * kWave), 0, stream, vals,
                     row_stride, N, k, out);
  return hipGetLastError();
}

}  // namespace sv
