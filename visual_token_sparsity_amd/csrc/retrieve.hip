// Query-aware retrieval for the decode stage: relevance scan + exact top-k.
//
// SparseVILA velog summary, Sec. 3.2 (Query-Aware Token Selection): the
// current query scores every cached vision token and only the top-k are
// activated.  xllm-io review, core formulas: TopK(Query . KV_Cache, k).
//
// Scan.  s[b,t] = sum_g qhat[b,g,:] . K[b,t,g,:] where qhat[b,g] is the sum of
// the query over the Tq query tokens and the G query heads sharing KV head g.
// The sum is linear, so summing the queries first gives the same score as
// summing per-head logits.  Decode is HBM-bound: every retained key row is
// read exactly once, as contiguous 16-byte vectors; a lane group of LPR lanes
// covers one token row (Hkv*D elements) and reduces it with cross-lane adds.
//
// Select.  One workgroup per row: four 8-bit radix passes over order-
// preserving uint32 keys find the k-th largest key T and how many keys equal
// to T are taken; a stable compaction then writes every key > T and the
// lowest-index keys == T, in ascending index order.  No global sort.
#include "common.h"

namespace sv {

// ----------------------------------------------------------------------------
// Scan
// ----------------------------------------------------------------------------
constexpr int kScanWaves = 4;

template <typename T, int CPL, int LPR>
__global__ __launch_bounds__(kScanWaves * kWave) void scan_kernel(
    const T* __restrict__ q, int Tq, int Hq, int G, const T* __restrict__ kv, int64_t bstride,
    int64_t tstride, int N, int D, float* __restrict__ scores) {
  constexpr int VE = Vec<T>::kElems;
  constexpr int RPW = kWave / LPR;  // rows per wave per step
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int b = blockIdx.y;
  const int sub = lane % LPR;
  const int rsub = lane / LPR;

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
        const T* qp = q + ((int64_t)(b * Tq + tau) * Hq + g * G + i) * D + d0;
        Vec<T> x;
        x.load(qp);
        float f[VE];
        x.to_f32(f);
#pragma unroll
        for (int v = 0; v < VE; ++v) qh[j][v] += f[v];
      }
    }
  }

  const T* base = kv + (int64_t)b * bstride;
  const int nwaves = gridDim.x * kScanWaves;
  for (int r0 = (blockIdx.x * kScanWaves + wave) * RPW; r0 < N; r0 += nwaves * RPW) {
    const int r = r0 + rsub;
    float acc = 0.f;
    if (r < N) {
      const T* row = base + (int64_t)r * tstride;
      Vec<T> x[CPL];
#pragma unroll
      for (int j = 0; j < CPL; ++j) x[j].load_stream(row + (sub + j * LPR) * VE);
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        float f[VE];
        x[j].to_f32(f);
#pragma unroll
        for (int v = 0; v < VE; ++v) acc = fmaf(qh[j][v], f[v], acc);
      }
    }
    acc = group_sum<LPR>(acc);
    if (r < N && sub == 0) scores[(int64_t)b * N + r] = acc;
  }
}

template <typename T, int CPL, int LPR>
static hipError_t scan_go(const void* q, int B, int Tq, int Hq, int G, const void* kv,
                          int64_t bs, int64_t ts, int N, int D, float* scores, hipStream_t st) {
  constexpr int RPW = kWave / LPR;
  const int rows_per_block = kScanWaves * RPW;
  int blocks = (N + rows_per_block - 1) / rows_per_block;
  const int cap = (8192 + B - 1) / B;  // enough waves in flight; the rest loop
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  dim3 grid(blocks, B);
  hipLaunchKernelGGL((scan_kernel<T, CPL, LPR>), grid, dim3(kScanWaves * kWave), 0, st,
                     (const T*)q, Tq, Hq, G, (const T*)kv, bs, ts, N, D, scores);
  return hipGetLastError();
}

template <typename T>
static hipError_t scan_dispatch(const void* q, int B, int Tq, int Hq, int G, const void* kv,
                                int64_t bs, int64_t ts, int N, int R, int D, float* scores,
                                hipStream_t st) {
  constexpr int VE = Vec<T>::kElems;
  const int C = R / VE;  // 16-byte chunks per token row
  // Each lane keeps CPL chunks of qhat; a row is covered by LPR = C / CPL lanes.
  switch (C) {
    case 8: return scan_go<T, 8, 1>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, st);
    case 16: return scan_go<T, 8, 2>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, st);
    case 32: return scan_go<T, 8, 4>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, st);
    case 64: return scan_go<T, 8, 8>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, st);
    case 128: return scan_go<T, 8, 16>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, st);
    case 256: return scan_go<T, 8, 32>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, st);
    case 512: return scan_go<T, 8, 64>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, st);
    case 1024: return scan_go<T, 16, 64>(q, B, Tq, Hq, G, kv, bs, ts, N, D, scores, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan(const void* q, int B, int Tq, int Hq, const void* kv, int64_t bstride,
                       int64_t tstride, int N, int Hkv, int D, int dtype, float* scores,
                       hipStream_t stream) {
  const int G = Hq / Hkv;
  const int R = Hkv * D;
  if (dtype == 1)
    return scan_dispatch<bf16_t>(q, B, Tq, Hq, G, kv, bstride, tstride, N, R, D, scores, stream);
  return scan_dispatch<float>(q, B, Tq, Hq, G, kv, bstride, tstride, N, R, D, scores, stream);
}

// ----------------------------------------------------------------------------
// Exact top-k per row
// ----------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

// Inclusive prefix sum over the block (all kSelThreads threads must call).
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* wsum,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  if (lane == kWave - 1) wsum[wave] = v;
  __syncthreads();
  if (wave == 0) {
    uint32_t w = lane < kSelWaves ? wsum[lane] : 0u;
#pragma unroll
    for (int off = 1; off < kSelWaves; off <<= 1) {
      const uint32_t o = __shfl_up(w, off, kWave);
      if (lane >= off) w += o;
    }
    if (lane < kSelWaves) wsum[lane] = w;  // inclusive wave totals
    if (lane == kSelWaves - 1) *total = w;
  }
  __syncthreads();
  const uint32_t before = wave > 0 ? wsum[wave - 1] : 0u;
  const uint32_t res = v + before;
  __syncthreads();  // wsum / total reusable after this
  return res;
}

__global__ __launch_bounds__(kSelThreads) void topk_rows_kernel(const float* __restrict__ vals,
                                                                int64_t row_stride, int N, int k,
                                                                int32_t* __restrict__ out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[kSelWaves];
  __shared__ uint32_t total;
  __shared__ uint32_t s_digit, s_above;
  const int tid = threadIdx.x;
  const float* v = vals + (int64_t)blockIdx.x * row_stride;
  int32_t* o = out + (int64_t)blockIdx.x * k;
  if (k <= 0) return;

  if (tid == 0) {
    s_digit = 0;
    s_above = 0;
  }
  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)k;  // how many still to take at/below the current prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += kSelThreads) {
      const uint32_t key = float_key(v[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // Suffix counts: bin (255 - tid) scanned in reversed order.
    const uint32_t c = tid < 256 ? hist[255 - tid] : 0u;
    const uint32_t incl = block_inclusive_scan(c, wsum, &total);  // # keys with digit >= 255-tid
    if (tid < 256) {
      const uint32_t excl = incl - c;  // # keys with digit > 255-tid
      if (excl < remaining && incl >= remaining) {
        s_digit = 255u - tid;
        s_above = excl;
      }
    }
    __syncthreads();
    remaining -= s_above;
    prefix |= s_digit << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t thr = prefix;  // the k-th largest key; take `remaining` keys equal to it

  uint32_t base_gt = 0, base_eq = 0;
  for (int t0 = 0; t0 < N; t0 += kSelThreads) {
    const int i = t0 + tid;
    uint32_t key = 0;
    if (i < N) key = float_key(v[i]);
    const uint32_t gt = (i < N && key > thr) ? 1u : 0u;
    const uint32_t eq = (i < N && key == thr) ? 1u : 0u;
    // gt count in the high half, eq count in the low half (a tile holds <= 1024 of each)
    const uint32_t packed = (gt << 16) | eq;
    const uint32_t incl = block_inclusive_scan(packed, wsum, &total);
    const uint32_t ex = incl - packed;
    const uint32_t ex_gt = base_gt + (ex >> 16), ex_eq = base_eq + (ex & 0xffffu);
    if (gt || (eq && ex_eq < remaining)) {
      const uint32_t pos = ex_gt + (ex_eq < remaining ? ex_eq : remaining);
      if (pos < (uint32_t)k) o[pos] = i;  // always true when the threshold is right
    }
    const uint32_t tot = total;
    base_gt += tot >> 16;
    base_eq += tot & 0xffffu;
    __syncthreads();
  }
}

hipError_t launch_topk_rows(const float* vals, int rows, int64_t row_stride, int N, int k,
                            int32_t* out, hipStream_t stream) {
  if (k <= 0 || rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_rows_kernel, dim3(rows), dim3(kSelThreads), 0, stream, vals,
                     row_stride, N, k, out);
  return hipGetLastError();
}

}  // namespace sv
