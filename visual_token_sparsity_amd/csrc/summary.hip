// Summary-token salience for prefill pruning: SparseVILA velog summary,
// Sec. 3.1, salience table (CLIP: the attention through which each token
// feeds the one summary token; RADIO: that attention averaged over several
// summary tokens).  The summary tokens are the first S tokens of a frame;
// their softmax rows over all N tokens are averaged over the summary tokens
// and the heads.
//
// summary_cols_kernel: one workgroup per (frame, head).  It holds the S
// summary queries (fp32, pre-scaled into base 2) and the S x N logits in
// LDS; each thread scores whole key rows (16-byte loads of one contiguous
// row), each wave then reduces whole logit rows (max, then the sum of
// exponentials), and each thread finally sums its columns' probabilities
// over the summary rows.  The per-head column values go to a workspace and
// summary_mean_kernel averages them over the heads in a fixed order, so the
// result does not depend on scheduling.  The keys are read once: the work is
// HBM-bound (about S*2 flops per key byte).
#include "summary.h"

namespace sv {

namespace {

constexpr int kSumThreads = 256;
constexpr int kSumCols = kSummaryMaxN / kSumThreads;  // columns per thread
constexpr int kSumMaxChunks = 16;                      // 16-byte chunks of a key row (D <= 128)

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Logits of every key row when D/8 = G is a power of two (used for S = 1, where
// it measured faster; with four summary rows the per-row reductions cost more
// than the coalescing gains): G consecutive lanes
// share a key row, one 16-byte chunk each, so every wave load is one
// contiguous 1 KB run; a shuffle reduction over the G lanes completes each
// dot product.  U chunks per lane are in flight per pass.
template <int G>
__device__ __forceinline__ void score_grouped(const uint16_t* __restrict__ kh, const float* qf,
                                              float* z, int N, int D, int S, int tid) {
  constexpr int U = 4;
  const uint4* kc = reinterpret_cast<const uint4*>(kh);
  const int total = N * G;               // 16-byte chunks of the frame-head's keys
  const int c = tid % G;                 // this lane's chunk within a row (fixed)
  for (int base = 0; base < total; base += kSumThreads * U) {   // uniform trip count
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = base + u * kSumThreads + tid;
      w[u] = e < total ? kc[e] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = base + u * kSumThreads + tid;
      const float kv[8] = {bf16_lo(w[u].x), bf16_hi(w[u].x), bf16_lo(w[u].y), bf16_hi(w[u].y),
                           bf16_lo(w[u].z), bf16_hi(w[u].z), bf16_lo(w[u].w), bf16_hi(w[u].w)};
      for (int s = 0; s < S; ++s) {
        const float* qs = qf + s * D + c * 8;
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) p = fmaf(qs[i], kv[i], p);
#pragma unroll
        for (int o = G / 2; o >= 1; o >>= 1) p += __shfl_xor(p, o, kWave);
        if (c == 0 && e < total) z[s * N + e / G] = p;
      }
    }
  }
}

__global__ __launch_bounds__(kSumThreads) void summary_cols_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int N, int D, int S,
    float qscale, float* __restrict__ colh) {
  extern __shared__ __align__(16) float sm[];
  float* z = sm;                          // [S][N] logits (base 2)
  float* qf = z + S * N;                  // [S][D] scaled queries
  float* rmax = qf + S * D;               // [S]
  float* rinv = rmax + kSummaryMaxS;      // [S]
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const size_t item = blockIdx.x;         // f * H + h
  const uint16_t* qh = q + item * (size_t)N * D;
  const uint16_t* kh = k + item * (size_t)N * D;

  for (int e = tid; e < S * D; e += kSumThreads) qf[e] = bf16_lo(qh[e]) * qscale;
  __syncthreads();

  // One summary row (CLIP): lane groups per key row, coalesced.  Several
  // rows: a key row per lane, whose loads serve all S dot products without
  // a reduction per row.
  const int D8 = D / 8;
  const bool grouped = S == 1 && (D8 == 1 || D8 == 2 || D8 == 4 || D8 == 8 || D8 == 16);
  if (grouped) switch (D8) {
    case 1: score_grouped<1>(kh, qf, z, N, D, S, tid); break;
    case 2: score_grouped<2>(kh, qf, z, N, D, S, tid); break;
    case 4: score_grouped<4>(kh, qf, z, N, D, S, tid); break;
    case 8: score_grouped<8>(kh, qf, z, N, D, S, tid); break;
    case 16: score_grouped<16>(kh, qf, z, N, D, S, tid); break;
    default: break;
  }
  for (int j = grouped ? N : tid; j < N; j += kSumThreads) {   // otherwise: a row per lane
    float acc[kSummaryMaxS];
#pragma unroll
    for (int s = 0; s < kSummaryMaxS; ++s) acc[s] = 0.f;
    // The whole key row's loads go out before any arithmetic.
    const uint4* kr = reinterpret_cast<const uint4*>(kh + (size_t)j * D);
    uint4 kw[kSumMaxChunks];
#pragma unroll
    for (int c = 0; c < kSumMaxChunks; ++c)
      if (c < D8) kw[c] = kr[c];
#pragma unroll
    for (int c = 0; c < kSumMaxChunks; ++c) {
      if (c < D8) {
        const uint4 w = kw[c];
        const float kv[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                             bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
        for (int s = 0; s < S; ++s) {
          const float* qs = qf + s * D + c * 8;
          float a = acc[s];
#pragma unroll
          for (int e = 0; e < 8; ++e) a = fmaf(qs[e], kv[e], a);
          acc[s] = a;
        }
      }
    }
#pragma unroll
    for (int s = 0; s < kSummaryMaxS; ++s)
      if (s < S) z[s * N + j] = acc[s];
  }
  __syncthreads();

  for (int s = wave; s < S; s += kSumThreads / kWave) {
    const float* zs = z + s * N;
    float m = -INFINITY;
    for (int j = lane; j < N; j += kWave) m = fmaxf(m, zs[j]);
    m = wave_max_f(m);
    float l = 0.f;
    for (int j = lane; j < N; j += kWave) l += exp2f(zs[j] - m);
    l = wave_sum_f(l);
    if (lane == 0) {
      rmax[s] = m;
      rinv[s] = 1.f / ((float)S * l);
    }
  }
  __syncthreads();

  float* out = colh + item * (size_t)N;
#pragma unroll
  for (int i = 0; i < kSumCols; ++i) {
    const int j = tid + i * kSumThreads;
    if (j < N) {
      float a = 0.f;
      for (int s = 0; s < S; ++s) a += exp2f(z[s * N + j] - rmax[s]) * rinv[s];
      out[j] = a;
    }
  }
}

__global__ __launch_bounds__(kSumThreads) void summary_mean_kernel(const float* __restrict__ colh,
                                                                   int H, int N, float inv_h,
                                                                   float* __restrict__ sal) {
  const int f = blockIdx.y;
  const int j = blockIdx.x * kSumThreads + threadIdx.x;
  if (j >= N) return;
  const float* c = colh + (size_t)f * H * N + j;
  float a = 0.f;
  for (int h = 0; h < H; ++h) a += c[(size_t)h * N];
  sal[(size_t)f * N + j] = a * inv_h;
}

}  // namespace

hipError_t launch_summary_salience(const void* q, const void* k, int F, int H, int N, int D, int S,
                                   float scale, int keep, float* colh_ws, float* sal,
                                   int32_t* idx_out, hipStream_t stream) {
  const size_t lds = ((size_t)S * N + (size_t)S * D + 2 * kSummaryMaxS) * sizeof(float);
  hipLaunchKernelGGL(summary_cols_kernel, dim3((unsigned)((int64_t)F * H)), dim3(kSumThreads), lds,
                     stream, (const uint16_t*)q, (const uint16_t*)k, N, D, S,
                     scale * 1.4426950408889634f, colh_ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(summary_mean_kernel, dim3((N + kSumThreads - 1) / kSumThreads, F),
                     dim3(kSumThreads), 0, stream, colh_ws, H, N, 1.0f / (float)H, sal);
  e = hipGetLastError();
  if (e != hipSuccess || keep <= 0) return e;
  return launch_topk_rows(sal, F, N, N, keep, idx_out, stream);
}

}  // namespace sv
