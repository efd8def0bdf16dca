// Query-agnostic salience for the prefill stage (no summary token).
//
// SparseVILA velog summary, Sec. 3.1: for encoders without a summary token
// (SigLIP, QwenVL) a token's salience is the intra-visual attention averaged
// over all tokens, and the same section's kernel streams the softmax
// normalisation and the salience accumulation so the attention matrix is
// never materialised.  xllm-io review, core formulas (salience), read as the
// attention each token receives.
//
// Per (frame, head) one workgroup of 8 waves.  The head's keys sit in LDS for
// the whole workgroup.  Waves form 4 pairs; a pair owns a 16-row block of
// queries at a time and each wave of the pair owns half of the columns, so a
// wave holds 16 rows x (16*TPW) columns of S = Q K^T in MFMA accumulators
// (bf16 inputs, fp32 accumulate, v_mfma_f32_16x16x32_bf16).  The row softmax
// is finished in registers: each wave reduces its half-row max and sum, the
// pair swaps (max, sum) through LDS, and every probability is added into a
// per-lane column accumulator with weight 2^((m_w - M) c) / L.  The exp is
// taken once per element, in base 2 (the scale is folded into c = scale *
// log2(e)).  Column sums of each (frame, head) go to the workspace; a second
// kernel averages them over heads and a third keeps the top tokens per frame.
#include "common.h"

namespace sv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kSalWaves = 8;
constexpr int kSalPairs = kSalWaves / 2;
constexpr int kSalXchFloats = 2 * kSalPairs * 2 * 16 * 2;  // [buf][pair][half][row][m,l]
constexpr int kSalMaxLds = 160 * 1024;

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16_t* p) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
}

template <int TPW, int KS>
__global__ __launch_bounds__(kSalWaves* kWave, 1) void salience_colsum_kernel(
    const bf16_t* __restrict__ Qg, const bf16_t* __restrict__ Kg, int N, int D, float c2,
    float* __restrict__ colsum) {
  extern __shared__ uint4 smem_u4[];
  constexpr int Ncp = 2 * TPW * 16;  // padded columns held in LDS
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem_u4);
  float* xch = reinterpret_cast<float*>(sK + Ncp * D);

  const int tid = threadIdx.x;
  const int64_t fh = blockIdx.x;
  const bf16_t* q = Qg + fh * N * D;
  const bf16_t* kk = Kg + fh * N * D;

  // Keys -> LDS, rows >= N zero-filled.
  const int chunks = Ncp * D / 8;
  for (int c = tid; c < chunks; c += kSalWaves * kWave) {
    const int row = (c * 8) / D;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < N) v = *reinterpret_cast<const uint4*>(kk + (int64_t)c * 8);
    reinterpret_cast<uint4*>(sK)[c] = v;
  }
  __syncthreads();

  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int pair = wave >> 1, half = wave & 1;
  const int li = lane & 15, lg = lane >> 4;
  const int tile0 = half * TPW;
  const int RB = (N + 15) / 16;
  const int iters = (RB + kSalPairs - 1) / kSalPairs;

  float colacc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) colacc[t] = 0.f;

  int buf = 0;
  for (int it = 0; it < iters; ++it) {
    const int rb = pair + kSalPairs * it;
    const bool active = rb < RB;
    f32x4 acc[TPW];
    float mx[4], sm[4];
    if (active) {
      const int qrow = rb * 16 + li;
      bf16x8 a[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int dd = 32 * s + 8 * lg;
        a[s] = (qrow < N && dd < D) ? load_bf16x8(q + (int64_t)qrow * D + dd) : zero_bf16x8();
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int col = (tile0 + t) * 16 + li;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const int dd = 32 * s + 8 * lg;
          const bf16x8 bv = dd < D ? load_bf16x8(sK + col * D + dd) : zero_bf16x8();
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], bv, acc[t], 0, 0, 0);
        }
      }
      // acc[t][r] = S[row 16*rb + 4*lg + r][col 16*(tile0+t) + li]; mask padded columns.
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        if ((tile0 + t) * 16 + li >= N) acc[t] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = -INFINITY;
#pragma unroll
        for (int t = 0; t < TPW; ++t) m = fmaxf(m, acc[t][r]);
        mx[r] = group_max<16>(m);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ms = mx[r] == -INFINITY ? 0.f : mx[r] * c2;
        float s = 0.f;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const float p = fast_exp2(fmaf(acc[t][r], c2, -ms));
          acc[t][r] = p;
          s += p;
        }
        sm[r] = group_sum<16>(s);
      }
      if (li == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* x = xch + ((((buf * kSalPairs + pair) * 2 + half) * 16) + 4 * lg + r) * 2;
          x[0] = mx[r];
          x[1] = sm[r];
        }
      }
    }
    __syncthreads();
    if (active) {
      float f[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float* x = xch + ((((buf * kSalPairs + pair) * 2 + (1 - half)) * 16) + 4 * lg + r) * 2;
        const float mo = x[0], lo = x[1];
        const float M = fmaxf(mx[r], mo);
        const float a_own = mx[r] == -INFINITY ? 0.f : fast_exp2((mx[r] - M) * c2);
        const float a_oth = mo == -INFINITY ? 0.f : fast_exp2((mo - M) * c2);
        const float L = sm[r] * a_own + lo * a_oth;
        const int row = rb * 16 + 4 * lg + r;
        f[r] = (row < N && L > 0.f) ? a_own / L : 0.f;
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        float c = colacc[t];
        c = fmaf(acc[t][0], f[0], c);
        c = fmaf(acc[t][1], f[1], c);
        c = fmaf(acc[t][2], f[2], c);
        c = fmaf(acc[t][3], f[3], c);
        colacc[t] = c;
      }
    }
    buf ^= 1;
  }

  // Column totals: lanes li, li+16, li+32, li+48 hold the same column.
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float c = colacc[t];
    c += __shfl_xor(c, 16, kWave);
    c += __shfl_xor(c, 32, kWave);
    colacc[t] = c;
  }
  __syncthreads();  // every wave is done reading sK; reuse it for the pair reduction
  float* red = reinterpret_cast<float*>(sK);  // [pair][Ncp]
  if (lg == 0) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) red[pair * Ncp + (tile0 + t) * 16 + li] = colacc[t];
  }
  __syncthreads();
  for (int j = tid; j < N; j += kSalWaves * kWave) {
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < kSalPairs; ++p) s += red[p * Ncp + j];
    colsum[fh * N + j] = s;
  }
}

// sal[f][j] = (1 / (H*N)) * sum_h colsum[f][h][j]
__global__ __launch_bounds__(256) void salience_mean_kernel(const float* __restrict__ colsum,
                                                           int H, int N, float inv,
                                                           float* __restrict__ sal) {
  const int f = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= N) return;
  const float* c = colsum + (int64_t)f * H * N + j;
  float s = 0.f;
  for (int h = 0; h < H; ++h) s += c[(int64_t)h * N];
  sal[(int64_t)f * N + j] = s * inv;
}

static int pick_tpw(int N) {
  const int half = ((N + 15) / 16 + 1) / 2;
  const int opts[] = {4, 8, 12, 16, 23, 24};
  for (int o : opts)
    if (o >= half) return o;
  return -1;
}

static size_t sal_lds_bytes(int tpw, int D) {
  return (size_t)2 * tpw * 16 * D * 2 + kSalXchFloats * sizeof(float);
}

bool salience_supported(int N, int D) {
  if (N < 1 || D < 8 || D > 96 || D % 8) return false;
  const int tpw = pick_tpw(N);
  if (tpw < 0) return false;
  return sal_lds_bytes(tpw, D) <= (size_t)kSalMaxLds;
}

template <int TPW, int KS>
static hipError_t sal_go(const void* q, const void* k, int FH, int N, int D, float c2,
                         float* colsum, hipStream_t st) {
  const size_t lds = sal_lds_bytes(TPW, D);
  // Opt in to more than 64 KiB of dynamic LDS; if the runtime refuses, the
  // launch below reports the failure.
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)salience_colsum_kernel<TPW, KS>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, kSalMaxLds);
    (void)hipGetLastError();
    attr_set = true;
  }
  hipLaunchKernelGGL((salience_colsum_kernel<TPW, KS>), dim3(FH), dim3(kSalWaves * kWave), lds, st,
                     (const bf16_t*)q, (const bf16_t*)k, N, D, c2, colsum);
  return hipGetLastError();
}

template <int TPW>
static hipError_t sal_ks(const void* q, const void* k, int FH, int N, int D, float c2,
                         float* colsum, hipStream_t st) {
  switch ((D + 31) / 32) {
    case 1: return sal_go<TPW, 1>(q, k, FH, N, D, c2, colsum, st);
    case 2: return sal_go<TPW, 2>(q, k, FH, N, D, c2, colsum, st);
    case 3: return sal_go<TPW, 3>(q, k, FH, N, D, c2, colsum, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_salience(const void* q, const void* k, int F, int H, int N, int D, float scale,
                           float* colsum_ws, float* sal, hipStream_t st) {
  const float c2 = scale * 1.4426950408889634f;
  const int FH = F * H;
  hipError_t e;
  switch (pick_tpw(N)) {
    case 4: e = sal_ks<4>(q, k, FH, N, D, c2, colsum_ws, st); break;
    case 8: e = sal_ks<8>(q, k, FH, N, D, c2, colsum_ws, st); break;
    case 12: e = sal_ks<12>(q, k, FH, N, D, c2, colsum_ws, st); break;
    case 16: e = sal_ks<16>(q, k, FH, N, D, c2, colsum_ws, st); break;
    case 23: e = sal_ks<23>(q, k, FH, N, D, c2, colsum_ws, st); break;
    case 24: e = sal_ks<24>(q, k, FH, N, D, c2, colsum_ws, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  dim3 grid((N + 255) / 256, F);
  hipLaunchKernelGGL(salience_mean_kernel, grid, dim3(256), 0, st, colsum_ws, H, N,
                     1.0f / ((float)H * (float)N), sal);
  return hipGetLastError();
}

}  // namespace sv
