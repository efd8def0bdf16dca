// Query-agnostic salience for long frames: two streaming passes.
//
// SparseVILA velog summary, Sec. 3.1 (kernel paragraph): salience of an
// encoder without a summary token is the column mean of its attention map,
// and for long visual inputs (QwenVL-style encoders, tens of thousands of
// tokens in one attention) the kernel streams the softmax normalisation and
// the salience accumulation instead of materialising the N x N map; the
// sciencestack abstract page, Fig. 5(a), credits that kernel with its largest
// prefill gain on QwenVL-style encoders.  One head's keys no longer fit on
// chip, so the map is computed twice:
//
//   pass 1 (rows):    lse_i = log2 sum_j 2^(x_ij),  x_ij = scale log2(e) q_i . k_j
//   pass 2 (columns): c_j   = sum_i 2^(x_ij - lse_i)          (= sum_i A_ij)
//
// Both passes use bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate) with
// one operand stationary in registers and the other streamed through LDS in
// stages shared by the workgroup's four waves:
//   pass 1: a wave holds 4 blocks of 16 query rows (A fragments); stages of 64
//     keys (B fragments) stream through LDS.  Each lane keeps its own running
//     (max, sum) for its column of every tile (rescaled once per 4-key-tile
//     stage), so the row reduction across lanes happens once at the end.
//   pass 2: a wave holds 4 tiles of 16 keys (B fragments); stages of 64 query
//     rows (A fragments) and their lse stream through LDS, and each lane adds
//     the probabilities of its key column.
// Stages are double-buffered: the next stage's fragments are loaded into
// registers while the current one is multiplied, then written to the other
// LDS buffer.  Fragments sit in LDS fragment-major (a wave's read of one
// 16x32 fragment is one contiguous 1 KB run: no bank conflicts).
//
// Padding: dims past D are zero on the stationary side (the streamed side
// loads clamped, finite data there); keys past N get x = -inf in pass 1 and
// no column in pass 2; rows past N get lse = +inf in pass 2 (probability 0).
#include "common.h"

namespace sv {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kStrWaves = 4;
constexpr int kStrThreads = kStrWaves * kWave;
constexpr int kStrTiles = 4;               // 16-wide tiles per wave (rows or keys)
constexpr int kStrBlock = kStrWaves * kStrTiles * 16;   // 256 rows / keys per workgroup
constexpr int kStrStage = kStrTiles * 16;  // 64 keys / rows per LDS stage
constexpr float kLag = 8.f;                // pass 1: most the shift may trail the row maximum

__device__ __forceinline__ bf16x8_t ld_frag(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16x8_t zero_frag() {
  return __builtin_bit_cast(bf16x8_t, make_uint4(0u, 0u, 0u, 0u));
}

template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Stage loader: the 64 rows [r0, r0 + 64) of one (frame, head) matrix as
// fragments, kStrTiles tiles x KS 32-wide steps of 1 KB each.  Thread tid
// carries chunks tid, tid + 256, ... of the stage (KS per thread), chunk f
// being tile t, step s, lane l = 16 lg + li: row r0 + 16 t + li, dims
// 32 s + 8 lg.  Rows past N read row N - 1 and dims past D read dims D - 8
// (finite data; the caller makes them count zero).
template <int KS>
__device__ __forceinline__ void stage_load(u32x4 (&v)[KS], const bf16_t* base, int N, int D,
                                           int r0) {
#pragma unroll
  for (int i = 0; i < KS; ++i) {
    const int f = i * kStrThreads + (int)threadIdx.x;
    const int l = f & (kWave - 1), ts = f / kWave;
    const int t = ts / KS, s = ts - t * KS;
    int row = r0 + 16 * t + (l & 15);
    row = row < N ? row : N - 1;
    int dd = 32 * s + 8 * (l >> 4);
    dd = dd < D ? dd : D - 8;
    v[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)row * D + dd);
  }
}
template <int KS>
__device__ __forceinline__ void stage_store(const u32x4 (&v)[KS], u32x4* lds) {
#pragma unroll
  for (int i = 0; i < KS; ++i) lds[i * kStrThreads + threadIdx.x] = v[i];
}
template <int KS>
constexpr int stage_chunks() { return kStrTiles * KS * kWave; }

// Pass 1: lse of every query row, in log2 units of the scaled logits.
template <int KS>
__global__ __launch_bounds__(kStrThreads) void salience_rowstat_kernel(
    const bf16_t* __restrict__ Qg, const bf16_t* __restrict__ Kg, int N, int D, int nblk,
    float c2, float* __restrict__ lse) {
  __shared__ u32x4 stage[2][stage_chunks<KS>()];
  const int64_t item = blockIdx.x / nblk;
  const int row0 = (blockIdx.x - (int)(item * nblk)) * kStrBlock;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int li = lane & 15, lg = lane >> 4;
  const bf16_t* q = Qg + item * (int64_t)N * D;
  const bf16_t* k = Kg + item * (int64_t)N * D;

  // This wave's query rows: A fragments of 4 row blocks, zero past D and N.
  bf16x8_t af[kStrTiles][KS];
#pragma unroll
  for (int rb = 0; rb < kStrTiles; ++rb) {
    const int row = row0 + (wave * kStrTiles + rb) * 16 + li;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int dd = 32 * s + 8 * lg;
      af[rb][s] = (row < N && dd < D) ? ld_frag(q + (int64_t)row * D + dd) : zero_frag();
    }
  }
  // Lane-local running max and sum for rows 16 rb + 4 lg + r over this lane's
  // key columns (column li of every tile).
  float m[kStrTiles][4], l[kStrTiles][4];
#pragma unroll
  for (int rb = 0; rb < kStrTiles; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m[rb][r] = -INFINITY;
      l[rb][r] = 0.f;
    }

  u32x4 pf[KS];
  const int nst = (N + kStrStage - 1) / kStrStage;
  stage_load<KS>(pf, k, N, D, 0);
  stage_store<KS>(pf, stage[0]);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    if (st + 1 < nst) stage_load<KS>(pf, k, N, D, (st + 1) * kStrStage);  // in flight during the MFMAs
    const bf16x8_t* frag = reinterpret_cast<const bf16x8_t*>(stage[cur]);
    f32x4_t S[kStrTiles][kStrTiles];  // [key tile][row block]
#pragma unroll
    for (int t = 0; t < kStrTiles; ++t) {
      bf16x8_t bk[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) bk[s] = frag[(t * KS + s) * kWave + lane];
#pragma unroll
      for (int rb = 0; rb < kStrTiles; ++rb) {
        f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rb][s], bk[s], a, 0, 0, 0);
        S[t][rb] = a;
      }
    }
    // Columns past N do not exist (the tail stage only).
    const int kcol = st * kStrStage + li;
    if (st + 1 < nst || N % kStrStage == 0) {
      // Every column counts.  The shift m lags the running maximum by at most
      // kLag (log2 units): it moves only when a stage's maximum rises past
      // m + kLag, so most stages take one max, one fma, one exp and one add
      // per element (terms stay below 2^kLag, and none underflows earlier
      // than with the exact running maximum).
#pragma unroll
      for (int rb = 0; rb < kStrTiles; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float smax = S[0][rb][r];
#pragma unroll
          for (int t = 1; t < kStrTiles; ++t) smax = fmaxf(smax, S[t][rb][r]);
          const float xm = smax * c2;
          float mm = m[rb][r], ll = l[rb][r];
          if (xm > mm + kLag) {  // also the first stage (m = -inf)
            ll = mm == -INFINITY ? 0.f : ll * fast_exp2(mm - xm);
            mm = xm;
          }
#pragma unroll
          for (int t = 0; t < kStrTiles; ++t) ll += fast_exp2(fmaf(S[t][rb][r], c2, -mm));
          l[rb][r] = ll;
          m[rb][r] = mm;
        }
      }
    } else {
      bool valid[kStrTiles];
#pragma unroll
      for (int t = 0; t < kStrTiles; ++t) valid[t] = kcol + 16 * t < N;
#pragma unroll
      for (int rb = 0; rb < kStrTiles; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x[kStrTiles];
          float mx = m[rb][r];
#pragma unroll
          for (int t = 0; t < kStrTiles; ++t) {
            x[t] = valid[t] ? S[t][rb][r] * c2 : -INFINITY;
            mx = fmaxf(mx, x[t]);
          }
          if (mx != -INFINITY) {
            float sum = l[rb][r] * fast_exp2(m[rb][r] - mx);  // m = -inf -> 0
#pragma unroll
            for (int t = 0; t < kStrTiles; ++t) sum += fast_exp2(x[t] - mx);
            l[rb][r] = sum;
            m[rb][r] = mx;
          }
        }
      }
    }
    if (st + 1 < nst) stage_store<KS>(pf, stage[cur ^ 1]);  // the other buffer: last read two stages ago
    __syncthreads();
  }

  // Combine the 16 lanes of each row: M = max m, L = sum l 2^(m - M).
#pragma unroll
  for (int rb = 0; rb < kStrTiles; ++rb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float M = m[rb][r];
      M = fmaxf(M, dpp_row<0xB1>(M));
      M = fmaxf(M, dpp_row<0x4E>(M));
      M = fmaxf(M, dpp_row<0x141>(M));
      M = fmaxf(M, dpp_row<0x140>(M));
      float L = m[rb][r] == -INFINITY ? 0.f : l[rb][r] * fast_exp2(m[rb][r] - M);
      L += dpp_row<0xB1>(L);
      L += dpp_row<0x4E>(L);
      L += dpp_row<0x141>(L);
      L += dpp_row<0x140>(L);
      const int row = row0 + (wave * kStrTiles + rb) * 16 + 4 * lg + r;
      if (li == 0 && row < N) lse[item * (int64_t)N + row] = M + __log2f(L);
    }
  }
}

// Pass 2: column sums c_j = sum_i 2^(x_ij - lse_i) of every key.
template <int KS>
__global__ __launch_bounds__(kStrThreads) void salience_colstream_kernel(
    const bf16_t* __restrict__ Qg, const bf16_t* __restrict__ Kg, int N, int D, int nblk,
    float c2, const float* __restrict__ lse, float* __restrict__ colsum) {
  __shared__ u32x4 stage[2][stage_chunks<KS>()];
  __shared__ __align__(16) float slse[2][kStrStage];
  const int64_t item = blockIdx.x / nblk;
  const int col0 = (blockIdx.x - (int)(item * nblk)) * kStrBlock;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int li = lane & 15, lg = lane >> 4;
  const bf16_t* q = Qg + item * (int64_t)N * D;
  const bf16_t* k = Kg + item * (int64_t)N * D;
  const float* ls = lse + item * (int64_t)N;

  // This wave's keys: B fragments of 4 tiles, zero past D (keys past N load
  // row N - 1 and are never written out).
  bf16x8_t bk[kStrTiles][KS];
#pragma unroll
  for (int t = 0; t < kStrTiles; ++t) {
    int key = col0 + (wave * kStrTiles + t) * 16 + li;
    key = key < N ? key : N - 1;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int dd = 32 * s + 8 * lg;
      bk[t][s] = dd < D ? ld_frag(k + (int64_t)key * D + dd) : zero_frag();
    }
  }
  float acc[kStrTiles];
#pragma unroll
  for (int t = 0; t < kStrTiles; ++t) acc[t] = 0.f;

  u32x4 pf[KS];
  const int nst = (N + kStrStage - 1) / kStrStage;
  auto load_lse = [&](int r0) {
    const int r = r0 + (int)threadIdx.x;
    return r < N ? ls[r] : INFINITY;  // rows past N: probability 0
  };
  stage_load<KS>(pf, q, N, D, 0);
  stage_store<KS>(pf, stage[0]);
  if (threadIdx.x < kStrStage) slse[0][threadIdx.x] = load_lse(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    float nl = 0.f;
    if (st + 1 < nst) {
      stage_load<KS>(pf, q, N, D, (st + 1) * kStrStage);
      if (threadIdx.x < kStrStage) nl = load_lse((st + 1) * kStrStage);
    }
    const bf16x8_t* frag = reinterpret_cast<const bf16x8_t*>(stage[cur]);
#pragma unroll
    for (int rt = 0; rt < kStrTiles; ++rt) {
      bf16x8_t a[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) a[s] = frag[(rt * KS + s) * kWave + lane];
      const f32x4_t L = *reinterpret_cast<const f32x4_t*>(&slse[cur][16 * rt + 4 * lg]);
#pragma unroll
      for (int t = 0; t < kStrTiles; ++t) {
        f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], bk[t][s], x, 0, 0, 0);
        // x[r] = S[row 16 rt + 4 lg + r][key 16 t + li]
        float p = fast_exp2(fmaf(x[0], c2, -L[0]));
        p += fast_exp2(fmaf(x[1], c2, -L[1]));
        p += fast_exp2(fmaf(x[2], c2, -L[2]));
        p += fast_exp2(fmaf(x[3], c2, -L[3]));
        acc[t] += p;
      }
    }
    if (st + 1 < nst) {
      stage_store<KS>(pf, stage[cur ^ 1]);
      if (threadIdx.x < kStrStage) slse[cur ^ 1][threadIdx.x] = nl;
    }
    __syncthreads();
  }
  // Lanes li, li + 16, li + 32, li + 48 hold the same key column.
#pragma unroll
  for (int t = 0; t < kStrTiles; ++t) {
    float c = acc[t];
    c += __shfl_xor(c, 16, kWave);
    c += __shfl_xor(c, 32, kWave);
    const int key = col0 + (wave * kStrTiles + t) * 16 + li;
    if (lg == 0 && key < N) colsum[item * (int64_t)N + key] = c;
  }
}

template <int KS>
hipError_t stream_go(const void* q, const void* k, int FH, int N, int D, float c2, float* lse,
                     float* colsum, hipStream_t st) {
  const int nblk = (N + kStrBlock - 1) / kStrBlock;
  const int64_t grid = (int64_t)FH * nblk;
  if (grid > 2147483647LL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(salience_rowstat_kernel<KS>, dim3((unsigned)grid), dim3(kStrThreads), 0, st,
                     (const bf16_t*)q, (const bf16_t*)k, N, D, nblk, c2, lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(salience_colstream_kernel<KS>, dim3((unsigned)grid), dim3(kStrThreads), 0, st,
                     (const bf16_t*)q, (const bf16_t*)k, N, D, nblk, c2, (const float*)lse, colsum);
  return hipGetLastError();
}

}  // namespace

bool salience_stream_supported(int N, int D) { return N >= 1 && D >= 8 && D <= 128 && D % 8 == 0; }

hipError_t launch_salience_stream(const void* q, const void* k, int FH, int N, int D, float c2,
                                  float* lse_ws, float* colsum_ws, hipStream_t st) {
  switch ((D + 31) / 32) {
    case 1: return stream_go<1>(q, k, FH, N, D, c2, lse_ws, colsum_ws, st);
    case 2: return stream_go<2>(q, k, FH, N, D, c2, lse_ws, colsum_ws, st);
    case 3: return stream_go<3>(q, k, FH, N, D, c2, lse_ws, colsum_ws, st);
    case 4: return stream_go<4>(q, k, FH, N, D, c2, lse_ws, colsum_ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sv
