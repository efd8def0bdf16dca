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

// ----------------------------------------------------------------------------
// Persistent column-stationary variant for the common head dims
// (D in {64, 72, 80, 96}).
//
// One workgroup of 8 waves per CU loops over (frame, head) items.  Wave w
// owns a fixed eighth of the key columns: its MFMA B fragments (TPW tiles of
// 16 keys x ceil(D/32) 32-wide k-steps) stay in registers for
// the whole item, so the inner loop reads no LDS.  Query rows stream from
// global memory as A fragments, two 16-row blocks per iteration, loaded one
// iteration ahead.  The keys of the next item are copied into an LDS staging
// buffer with direct global->LDS loads while the current item is computed.
// A head dim that is not a multiple of 32 gets one more 32-wide step whose
// lanes beyond D feed zeros (one step shape for every D keeps the MFMA
// accumulation chains uniform).
//
// Row shift.  Softmax is shift-invariant, so any shift >= the row max works.
// The kernel uses the Cauchy-Schwarz bound c_i = |q_i| * max_j |k_j| * scale
// (in log2 units, times 1 + 2^-10 to cover rounding): every exponent is then
// <= 0 without a max pass, and the waves only have to add their partial row
// sums.  A row block whose bound exceeds 48 (the row maximum could sit below
// 2^-96) uses the exact maximum of each wave's columns instead, and the
// partial sums are then merged with max-rescaling.
// ----------------------------------------------------------------------------
constexpr int kColWaves = 8;  // waves per workgroup, each owning a column slice
constexpr int kRowBlocks = 1;  // 16-row blocks per iteration

__device__ __forceinline__ float sumsq8(const bf16x8& v) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = fmaf((float)v[i], (float)v[i], s);
  return s;
}

// Cross-lane steps inside a row of 16 lanes with DPP (VALU modifiers, no LDS trip).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Every lane gets the sum (or max) over its 16-lane row.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}

template <int D, int TPW>
__global__ __launch_bounds__(kColWaves* kWave, 1) void salience_colstat_kernel(
    const bf16_t* __restrict__ Qg, const bf16_t* __restrict__ Kg, int FH, int N, float c2,
    float* __restrict__ colsum, const int32_t* __restrict__ only) {
  // 32-wide k-steps; lanes whose 8-element chunk lies beyond D feed zeros.
  constexpr int KS = (D + 31) / 32;
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  static_assert(D % 8 == 0, "D must be a multiple of 8");
  constexpr int NT = kColWaves * kWave;
  constexpr int CPW = TPW * 16;               // columns per wave
  constexpr int Ncp = kColWaves * CPW;        // padded key rows in the staging buffer
  constexpr int RPI = kRowBlocks * 16;        // query rows per iteration
  extern __shared__ uint4 smem_u4[];
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem_u4);            // [Ncp][D] staged keys
  float* xch = reinterpret_cast<float*>(sK + Ncp * D);        // [2][RPI][2][kColWaves]
  float* qn2 = xch + 2 * RPI * 2 * kColWaves;                 // [Ncp] query-row norms |q_r|
  uint32_t* maxu = reinterpret_cast<uint32_t*>(qn2 + Ncp);    // [2][2] max |k|^2, max |q|^2
  uint32_t* arrived = maxu + 4;                                // partial-sum arrivals (bound loop)

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int li = lane & 15, lg = lane >> 4;
  const int c0 = wave * CPW;
  const int RB = (N + 15) / 16;
  const int iters = (RB + kRowBlocks - 1) / kRowBlocks;
  const int kbytes = N * D * 2;

  // Staging rows >= N stay zero for every item; so do their query norms.
  for (int c = N * D / 8 + tid; c < Ncp * D / 8; c += NT) smem_u4[c] = make_uint4(0, 0, 0, 0);
  if (tid < 5) maxu[tid] = 0u;  // key/query maxima of both parities, arrival counter
  // Direct global->LDS copy of one item's keys (1 KB per wave instruction).
  auto stage_keys = [&](int item) {
    const char* src = reinterpret_cast<const char*>(Kg + (int64_t)item * N * D);
    char* dst = reinterpret_cast<char*>(sK);
    for (int chunk = wave; chunk * 1024 < kbytes; chunk += kColWaves) {
      const int off = chunk * 1024 + lane * 16;
      if (off < kbytes)
        __builtin_amdgcn_global_load_lds(src + off, dst + chunk * 1024, 16, 0, 0);
    }
  };
  // Unconditional loads (no exec-masked branch, so no early vmcnt wait).  A
  // lane whose d-chunk lies beyond D may load any finite data because its key
  // partner is zero; a row beyond N loads row N-1 and uses that row's shift, so
  // its probabilities stay <= 1 and are dropped by a zero weight.
  auto load_a_raw = [&](const bf16_t* q, int rb, bf16x8 (&af)[KS]) {
    int row = rb * 16 + li;
    row = row < N ? row : N - 1;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int dd = 32 * s + 8 * lg;
      af[s] = load_bf16x8(q + (int64_t)row * D + (dd < D ? dd : 0));
    }
  };
  auto load_a = [&](const bf16_t* q, int rb, bf16x8 (&af)[KS]) {
    const int row = rb * 16 + li;
    const bool ok = rb < RB && row < N;
    const int64_t rowc = ok ? row : 0;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int dd = 32 * s + 8 * lg;
      const bool in = ok && dd < D;
      const uint4 u = *reinterpret_cast<const uint4*>(q + rowc * D + (dd < D ? dd : 0));
      af[s] = __builtin_bit_cast(bf16x8, in ? u : make_uint4(0, 0, 0, 0));
    }
  };
  auto scores = [&](const bf16x8 (&af)[KS], const bf16x8 (&bk)[TPW][KS], int t) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], bk[t][s], acc, 0, 0, 0);
    if (c0 + 16 * t + 16 > N && c0 + 16 * t + li >= N)  // padded key columns
      acc = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    return acc;
  };

  // With `only`, items whose flag is 0 are skipped (another kernel computed them).
  auto next_item = [&](int i) {
    if (only)
      while (i < FH && only[i] == 0) i += gridDim.x;
    return i;
  };
  int item = next_item(blockIdx.x);
  if (item < FH) stage_keys(item);
  int buf = 0, par = 0;
  for (int nxt; item < FH; item = nxt, par ^= 1) {
    wait_stores_complete();  // this wave's direct loads have landed (vmcnt = 0)
    __syncthreads();
    const bf16_t* q = Qg + (int64_t)item * N * D;

    // This wave's key fragments and the largest key norm; every query-row norm.
    bf16x8 bk[TPW][KS];
    float kn2 = 0.f;  // padded columns are zero
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int col = c0 + 16 * t + li;
      float n2 = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int dd = 32 * s + 8 * lg;
        bk[t][s] = dd < D ? load_bf16x8(sK + col * D + dd) : zero_bf16x8();
        n2 += sumsq8(bk[t][s]);
      }
      // the 4 lanes li, li+16, li+32, li+48 hold the chunks of one key row
      n2 += __shfl_xor(n2, 16, kWave);
      n2 += __shfl_xor(n2, 32, kWave);
      kn2 = fmaxf(kn2, n2);
    }
    float qmax2 = 0.f;
    for (int r = tid; r < N; r += NT) {
      float n2 = 0.f;
#pragma unroll
      for (int c = 0; c < CH; ++c) n2 += sumsq8(load_bf16x8(q + (int64_t)r * D + 8 * c));
      qn2[r] = __builtin_amdgcn_sqrtf(n2);  // |q_r|
      qmax2 = fmaxf(qmax2, n2);
    }
    kn2 = group_max<kWave>(kn2);
    qmax2 = group_max<kWave>(qmax2);
    // Rows N..Ncp-1 (padding of the last row block) reuse row N-1's norm.
    if (tid == 0) {
      float n2 = 0.f;
#pragma unroll
      for (int c = 0; c < CH; ++c) n2 += sumsq8(load_bf16x8(q + (int64_t)(N - 1) * D + 8 * c));
      const float nn = __builtin_amdgcn_sqrtf(n2);
      for (int r = N; r < Ncp; ++r) qn2[r] = nn;
    }
    if (lane == 0) {  // non-negative floats: uint order
      atomicMax(&maxu[2 * par], __float_as_uint(kn2));
      atomicMax(&maxu[2 * par + 1], __float_as_uint(qmax2));
    }
    __syncthreads();  // fragments are in registers: the staging buffer is free
    const float kc = __builtin_amdgcn_sqrtf(__uint_as_float(maxu[2 * par])) * c2 * 1.0009765625f;
    const float cmax = __builtin_amdgcn_sqrtf(__uint_as_float(maxu[2 * par + 1])) * kc;
    if (tid < 2) maxu[2 * (par ^ 1) + tid] = 0u;
    nxt = next_item(item + gridDim.x);
    if (nxt < FH) stage_keys(nxt);

    float colacc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) colacc[t] = 0.f;

    if (cmax <= 48.f) {
      // Bound shift for the whole item: c_i = |q_i| * max|k| * scale (log2 units).
      // Every wave uses the same shift for a row, so only partial sums are exchanged.
      // Software pipeline over iterations of kRowBlocks row blocks:
      //   MFMA(it) | column update of it-1 (independent, overlaps the MFMAs)
      //   exp(it) -> partial row sums -> LDS | barrier | 1/L(it)
      // Padded key columns (zero rows, so S = 0 exactly) each add exactly
      // 2^-c_i to a row sum; the lanes owning them subtract that instead of
      // masking every score.
      int npad = 0;
#pragma unroll
      for (int t = 0; t < TPW; ++t) npad += (c0 + 16 * t + li >= N) ? 1 : 0;
      const float fpad = (float)npad;
      const bool padw = __any(npad > 0);  // only the wave(s) owning columns >= N
      bf16x8 af[kRowBlocks][KS];
#pragma unroll
      for (int h = 0; h < kRowBlocks; ++h) load_a_raw(q, h, af[h]);

      auto mfma_phase = [&](f32x4 (&S)[kRowBlocks][TPW], int it) {
#pragma unroll
        for (int h = 0; h < kRowBlocks; ++h) {
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2)
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[h][s2], bk[t][s2], acc, 0, 0, 0);
            S[h][t] = acc;
          }
        }
        // The A fragments are consumed: the next row blocks load into the same registers.
#pragma unroll
        for (int h = 0; h < kRowBlocks; ++h) load_a_raw(q, kRowBlocks * (it + 1) + h, af[h]);
      };
      auto update_phase = [&](const f32x4 (&S)[kRowBlocks][TPW], const float (&f)[kRowBlocks][4]) {
#pragma unroll
        for (int h = 0; h < kRowBlocks; ++h) {
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
            float c = colacc[t];
            c = fmaf(S[h][t][0], f[h][0], c);
            c = fmaf(S[h][t][1], f[h][1], c);
            c = fmaf(S[h][t][2], f[h][2], c);
            c = fmaf(S[h][t][3], f[h][3], c);
            colacc[t] = c;
          }
        }
      };
      // exp + partial row sums of iteration it -> LDS, then this wave's arrival.
      auto publish = [&](f32x4 (&S)[kRowBlocks][TPW], int it) {
#pragma unroll
        for (int h = 0; h < kRowBlocks; ++h) {
          const int r0 = (kRowBlocks * it + h) * 16 + 4 * lg;
          const float4 n4 = *reinterpret_cast<const float4*>(qn2 + r0);
          const float cb[4] = {n4.x * kc, n4.y * kc, n4.z * kc, n4.w * kc};
          float part[4] = {0.f, 0.f, 0.f, 0.f};
          if (padw) {
#pragma unroll
            for (int r = 0; r < 4; ++r) part[r] = -fpad * fast_exp2(-cb[r]);
          }
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float p = fast_exp2(fmaf(S[h][t][r], c2, -cb[r]));
              S[h][t][r] = p;
              part[r] += p;
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) part[r] = row16_sum(part[r]);
          if (li == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              xch[((it & 1) * RPI + h * 16 + 4 * lg + r) * kColWaves + wave] = part[r];
          }
        }
        // LDS operations of one wave complete in order: the partials land before the count.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      };
      // Wait until all waves published iteration it, then the row weights 1/L.
      // Every wave publishes it before it waits on it-1, so the wait always ends;
      // the spin is bounded all the same.  Double-buffered partials are safe: a
      // wave overwrites buffer (it & 1) only after seeing every wave's it+1,
      // which each wave publishes after reading buffer (it & 1).
      auto collect = [&](int it, float (&f)[kRowBlocks][4]) {
        const uint32_t target = (uint32_t)kColWaves * (uint32_t)(it + 1);
        for (int spin = 0; spin < (1 << 22); ++spin) {
          if (__hip_atomic_load(arrived, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
          __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
        for (int h = 0; h < kRowBlocks; ++h) {
          // Lane (quad position r) sums the 8 wave partials of row 4*lg + r;
          // quad broadcasts then give every lane the weights of its 4 rows.
          const int r = li & 3;
          const float* x = xch + ((it & 1) * RPI + h * 16 + 4 * lg + r) * kColWaves;
          const float4 l0 = *reinterpret_cast<const float4*>(x);
          const float4 l1 = *reinterpret_cast<const float4*>(x + 4);
          const float L = ((l0.x + l0.y) + (l0.z + l0.w)) + ((l1.x + l1.y) + (l1.z + l1.w));
          const int row = (kRowBlocks * it + h) * 16 + 4 * lg + r;
          const float fr = row < N ? __builtin_amdgcn_rcpf(L) : 0.f;
          f[h][0] = dpp_f32<0x00>(fr);  // quad_perm [0,0,0,0]
          f[h][1] = dpp_f32<0x55>(fr);  // quad_perm [1,1,1,1]
          f[h][2] = dpp_f32<0xAA>(fr);  // quad_perm [2,2,2,2]
          f[h][3] = dpp_f32<0xFF>(fr);  // quad_perm [3,3,3,3]
        }
      };

      f32x4 SA[kRowBlocks][TPW], SB[kRowBlocks][TPW];
      float fA[kRowBlocks][4], fB[kRowBlocks][4];
      // MFMA(it) | wait for it-1's partials, weights, column update of it-1 | publish(it)
      mfma_phase(SA, 0);
      publish(SA, 0);
      int it = 1;
      for (; it + 1 < iters; it += 2) {
        mfma_phase(SB, it);
        collect(it - 1, fA);
        update_phase(SA, fA);
        publish(SB, it);
        mfma_phase(SA, it + 1);
        collect(it, fB);
        update_phase(SB, fB);
        publish(SA, it + 1);
      }
      if (it < iters) {
        mfma_phase(SB, it);
        collect(it - 1, fA);
        update_phase(SA, fA);
        publish(SB, it);
        collect(it, fB);
        update_phase(SB, fB);
      } else {
        collect(it - 1, fA);
        update_phase(SA, fA);
      }
      __syncthreads();  // every wave is done with the partials and the counter
      if (tid == 0) *arrived = 0u;  // ordered before the next publish by the item-start barrier
    } else {
      // Exact row max: each wave shifts by the max over its own columns and the
      // partial (max, sum) pairs are merged with max-rescaling.
      for (int it = 0; it < iters; ++it) {
        bf16x8 af[kRowBlocks][KS];
#pragma unroll
        for (int h = 0; h < kRowBlocks; ++h) load_a(q, kRowBlocks * it + h, af[h]);
        f32x4 S[kRowBlocks][TPW];
        float sh[kRowBlocks][4];
#pragma unroll
        for (int h = 0; h < kRowBlocks; ++h) {
#pragma unroll
          for (int t = 0; t < TPW; ++t) S[h][t] = scores(af[h], bk, t);
          float part[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float m = -INFINITY;
#pragma unroll
            for (int t = 0; t < TPW; ++t) m = fmaxf(m, S[h][t][r]);
            m = row16_max(m);
            sh[h][r] = m == -INFINITY ? -INFINITY : m * c2;
            const float base = m == -INFINITY ? 0.f : m * c2;
            float sum = 0.f;
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
              const float p = fast_exp2(fmaf(S[h][t][r], c2, -base));
              S[h][t][r] = p;
              sum += p;
            }
            part[r] = row16_sum(sum);
          }
          if (li == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float* x = xch + ((buf * RPI + h * 16 + 4 * lg + r) * 2) * kColWaves + wave;
              x[0] = sh[h][r];
              x[kColWaves] = part[r];
            }
          }
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < kRowBlocks; ++h) {
          float f[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float* x = xch + ((buf * RPI + h * 16 + 4 * lg + r) * 2) * kColWaves;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kColWaves; ++w) M = fmaxf(M, x[w]);
            float L = 0.f;
#pragma unroll
            for (int w = 0; w < kColWaves; ++w)
              L += x[w] == -INFINITY ? 0.f : x[kColWaves + w] * fast_exp2(x[w] - M);
            const float a_own = sh[h][r] == -INFINITY ? 0.f : fast_exp2(sh[h][r] - M);
            const int row = (kRowBlocks * it + h) * 16 + 4 * lg + r;
            f[r] = (row < N && L > 0.f) ? a_own / L : 0.f;
          }
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
            float c = colacc[t];
            c = fmaf(S[h][t][0], f[0], c);
            c = fmaf(S[h][t][1], f[1], c);
            c = fmaf(S[h][t][2], f[2], c);
            c = fmaf(S[h][t][3], f[3], c);
            colacc[t] = c;
          }
        }
        buf ^= 1;
      }
    }

    // Column totals: lanes li, li+16, li+32, li+48 hold the same column.
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      float c = colacc[t];
      c += __shfl_xor(c, 16, kWave);
      c += __shfl_xor(c, 32, kWave);
      const int col = c0 + 16 * t + li;
      if (lg == 0 && col < N) colsum[(int64_t)item * N + col] = c;
    }
  }
}

// ----------------------------------------------------------------------------
// Row-stationary variant with MFMA column sums (D in {64, 72, 80, 96}).
//
// One workgroup of 8 waves per CU loops over (frame, head) items.  The item's
// keys sit in LDS.  A wave owns a 16-row block of queries at a time and sweeps
// every key column itself, so a row's softmax denominator is complete inside
// the wave: no exchange between waves, no barrier per row block.
//
// Per 16x16 tile of S = Q K^T (bf16 MFMA, fp32 accumulate):
//     p = 2^(S * scale * log2(e) - b_i)          (one exp per element)
//     P tile kept in registers as fp16 (round to nearest even)
//     l_i += p, summed in fp32 over the rounded fp16 values
// After the sweep the row weights w_i = 1/l_i are known, and the column sums
// c_j += sum_i w_i p_ij are one fp16 MFMA per tile: the P tile, as it comes
// out of the score MFMA, is already the B operand of v_mfma_f32_16x16x16_f16
// with the 16 rows of the block as the reduction index; the A operand holds
// w split into an fp16 high part (row 0) and the fp16 residual (row 1).
//
// Shift b_i.  Softmax is shift-invariant.  b_i = |q_i| * max_j |k_j| * scale
// (log2 units, times 1 + 2^-10 for rounding) bounds |S_ij * scale| by
// Cauchy-Schwarz, so every exponent lies in [-2 b_i, 0].  With b_i <= 7 every
// p is a normal fp16 number, whose rounding (relative 2^-11) averages out
// over the rows of a column.  An item with a row above that bound is flagged
// and left to the fp32 column-stationary kernel, launched right after.
//
// The kernel is compiled for an exact tile count (ceil(N/16)), so only the
// last tile can hold columns >= N; their probabilities are set to zero there.
// ----------------------------------------------------------------------------
constexpr int kRowWaves = 8;
constexpr float kHalfBound = 7.f;  // b_i limit: p >= 2^-14, a normal fp16
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

__device__ __forceinline__ f16x4 pack_f16x4(float a, float b, float c, float d) {
  const f16x2 lo = __builtin_convertvector((f32x2){a, b}, f16x2);  // v_cvt_pk_f16_f32
  const f16x2 hi = __builtin_convertvector((f32x2){c, d}, f16x2);
  return f16x4{lo[0], lo[1], hi[0], hi[1]};
}

// Fragment-major key tiles: byte offset of k-step s inside a 16-key tile, and
// the number of 8-dim lane groups that step stores.
template <int D>
__device__ __forceinline__ int frag_step_off(int s) {
  return 16 * 2 * (32 * s < D ? 32 * s : D);
}
template <int D>
__device__ __forceinline__ int frag_step_nlg(int s) {
  const int r = (D - 32 * s) / 8;
  return r < 4 ? r : 4;
}

// With D = 32 m + 8 (D = 72) the last k-step carries one lane group of data
// (16 lanes x 16 bytes).  Its fragments are packed four tiles to a 1 KB
// block (lane group j holds tile 4 q + j), read once per four tiles; tile
// 4 q + j multiplies it with a query fragment whose data sits in lane group
// j (zeros elsewhere).  Group q of four tiles: [full k-steps of 4 tiles][tail].
__host__ __device__ constexpr bool rows_tail_pack(int D) { return D % 32 == 8; }
__host__ __device__ constexpr int rows_full_steps(int D) {
  return rows_tail_pack(D) ? D / 32 : (D + 31) / 32;
}
// Bytes of the keys region in LDS.
__host__ __device__ constexpr int rows_k_bytes(int D, int ntile) {
  return rows_tail_pack(D) ? ((ntile + 3) / 4) * (4 * (D / 32) * 1024 + 1024)
                           : ntile * 16 * D * 2 + 1024;
}

template <int D, int NTILE>
__global__ __launch_bounds__(kRowWaves* kWave, 1) void salience_rows_kernel(
    const bf16_t* __restrict__ Qg, const bf16_t* __restrict__ Kg, int FH, int N, float c2,
    float* __restrict__ colsum, int32_t* __restrict__ redo) {
  // 32-wide k-steps; lanes whose 8 dims lie beyond D get zero query data.
  constexpr int KS = (D + 31) / 32;
  constexpr bool TP = rows_tail_pack(D);  // packed last k-step (see rows_tail_pack)
  constexpr int KF = rows_full_steps(D);  // k-steps stored per tile
  constexpr int DT = 32 * KF;             // first dim of the packed step
  constexpr int NT = kRowWaves * kWave;
  constexpr int NC = NTILE * 16;  // key columns rounded up to whole tiles
  static_assert(D % 8 == 0, "D must be a multiple of 8");
  extern __shared__ uint4 smem_u4[];
  // Keys in LDS, fragment-major: tile t (16 keys, 16 * D * 2 bytes) holds,
  // for each 32-wide k-step s, the 16-byte B fragments of the lanes that carry
  // data (lg < nlg(s)), in lane order, so a wave's fragment read is one
  // contiguous run of 16-byte chunks (no bank conflicts).  A zeroed 1 KB pad
  // follows: a partial step's lanes past D read into the next tile or the pad,
  // finite values that meet zero query data.
  char* sK = reinterpret_cast<char*>(smem_u4);                         // keys (rows_k_bytes)
  float* cacc = reinterpret_cast<float*>(sK + rows_k_bytes(D, NTILE)); // [kRowWaves][NC] wave sums
  uint32_t* ctl = reinterpret_cast<uint32_t*>(cacc + kRowWaves * NC);  // max|k|^2, redo

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int li = lane & 15, lg = lane >> 4;
  const int RB = (N + 15) / 16;
  float* myacc = cacc + wave * NC;

  constexpr int TB = 16 * D * 2;            // bytes per key tile (unpacked)
  constexpr int FSB = KF * 1024;            // packed: full-step bytes per tile
  constexpr int GB = 4 * FSB + 1024;        // packed: bytes per group of four tiles
  constexpr int NG = (NTILE + 3) / 4;       // packed: groups
  // Byte offset of tile t's k-step s fragments, and of group q's tail block.
  auto frag_at = [&](int t, int s) {
    return TP ? (t / 4) * GB + (t % 4) * FSB + s * 1024 : t * TB + frag_step_off<D>(s);
  };
  auto tail_at = [&](int qg) { return qg * GB + 4 * FSB; };
  // Keys of rows N..NC-1 and the pad stay zero for every item (the staging
  // never writes them).
  for (int c = tid; c < rows_k_bytes(D, NTILE) / 16; c += NT) smem_u4[c] = make_uint4(0, 0, 0, 0);

  // A fragments of row block rb: lane (li, lg) holds row 16 rb + li, dims
  // 32 s + 8 lg .. +7.  Rows >= N and dims >= D read as zeros.
  // Packed tail (TP): af[KS-1] holds dims DT..DT+7 of row li in every lane;
  // tail_frags() then keeps them in lane group j only, for each j.
  auto load_a = [&](const bf16_t* q, int rb, bf16x8 (&af)[KS]) {
    const int row = rb * 16 + li;
    const bool ok = row < N;
    const int64_t rowc = ok ? row : 0;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int dd = (TP && s == KS - 1) ? DT : 32 * s + 8 * lg;
      const bool in = ok && dd < D;
      const uint4 u = *reinterpret_cast<const uint4*>(q + rowc * D + (dd < D ? dd : 0));
      af[s] = __builtin_bit_cast(bf16x8, in ? u : make_uint4(0, 0, 0, 0));
    }
  };
  auto tail_frags = [&](const bf16x8& raw, bf16x8 (&at)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) at[j] = lg == j ? raw : zero_bf16x8();
  };

  for (int item = blockIdx.x; item < FH; item += gridDim.x) {
    const bf16_t* q = Qg + (int64_t)item * N * D;
    bf16x8 af[KS];
    load_a(q, wave, af);  // in flight during the key staging
    float colacc[NTILE];  // this wave's column sums (lanes 0-15: column 16 t + li)
#pragma unroll
    for (int t = 0; t < NTILE; ++t) colacc[t] = 0.f;
    __syncthreads();      // the previous item is done with sK, cacc and ctl
    if (tid < 2) ctl[tid] = 0u;
    {
      // Direct global->LDS loads, one per (tile, k-step): lane (li, lg) fetches
      // row 16 t + li, dims 32 s + 8 lg .. +7, and lands in lane order.
      // Packed tail: one more load per group, lane (li, j) fetching row
      // 16 (4 q + j) + li, dims DT .. DT+7.
      const char* src = reinterpret_cast<const char*>(Kg + (int64_t)item * N * D);
      constexpr int JOBS = TP ? NG * (4 * KF + 1) : NTILE * KS;
      for (int f = wave; f < JOBS; f += kRowWaves) {
        int t, s2, dim, off;
        bool on;
        if (TP) {
          const int qg = f / (4 * KF + 1), r = f - qg * (4 * KF + 1);
          if (r < 4 * KF) {
            t = 4 * qg + r / KF;
            s2 = r % KF;
            dim = 32 * s2 + 8 * lg;
            off = frag_at(t, s2);
            on = t < NTILE;
          } else {
            t = 4 * qg + lg;
            s2 = KS - 1;
            dim = DT;
            off = tail_at(qg);
            on = t < NTILE;
          }
        } else {
          t = f / KS;
          s2 = f - t * KS;
          dim = 32 * s2 + 8 * lg;
          off = frag_at(t, s2);
          on = lg < frag_step_nlg<D>(s2);
        }
        const int row = 16 * t + li;
        if (on && row < N) {
          // (the LDS destination goes through a local: written inline as the
          // builtin's argument, the host pass dropped the kernel's stub)
          char* dst = sK + off;
          __builtin_amdgcn_global_load_lds(src + ((int64_t)row * D + dim) * 2, dst, 16, 0, 0);
        }
      }
    }
    wait_stores_complete();  // this wave's direct loads have landed (vmcnt = 0)
    __syncthreads();
    float kn2 = 0.f;
    for (int r = tid; r < N; r += NT) {
      const int t = r / 16, rl = r - 16 * t;
      float n2 = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < KF; ++s2)
        for (int g2 = 0; g2 < frag_step_nlg<D>(s2); ++g2)
          n2 += sumsq8(*reinterpret_cast<const bf16x8*>(sK + frag_at(t, s2) + (16 * g2 + rl) * 16));
      if (TP) n2 += sumsq8(*reinterpret_cast<const bf16x8*>(sK + tail_at(t / 4) + (16 * (t % 4) + rl) * 16));
      kn2 = fmaxf(kn2, n2);
    }
    kn2 = group_max<kWave>(kn2);
    if (lane == 0) atomicMax(&ctl[0], __float_as_uint(kn2));  // non-negative: uint order
    __syncthreads();
    const float kc = __builtin_amdgcn_sqrtf(__uint_as_float(ctl[0])) * c2 * 1.0009765625f;

    for (int rb = wave; rb < RB; rb += kRowWaves) {
      // |q|^2 of row li: the 4 lanes li + 16 lg hold its chunks (a packed
      // tail is in every lane: counted once).
      float n2 = 0.f;
#pragma unroll
      for (int s = 0; s < KF; ++s) n2 += sumsq8(af[s]);
      if (TP) n2 += lg == 0 ? sumsq8(af[KS - 1]) : 0.f;
      n2 += __shfl_xor(n2, 16, kWave);
      n2 += __shfl_xor(n2, 32, kWave);
      bf16x8 at[4];  // packed tail: query dims DT.. in lane group j only
      if (TP) tail_frags(af[KS - 1], at);
      // Output rows of this lane are 16 rb + 4 lg + r.
      float b[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) b[r] = __builtin_amdgcn_sqrtf(__shfl(n2, 4 * lg + r, kWave)) * kc;
      if (__any(fmaxf(fmaxf(b[0], b[1]), fmaxf(b[2], b[3])) > kHalfBound)) {
        if (lane == 0) ctl[1] = 1u;
      }
      bf16x8 an[KS];
      load_a(q, rb + kRowWaves, an);  // next row block (zeros past the end)

      // Software pipeline over column tiles: step t issues the LDS reads of
      // tile t+3 and the MFMAs of tile t+1, then the exps of tile t, so the
      // matrix core and the LDS work under the VALU.  A scheduling barrier
      // closes each step (it keeps the compiler from hoisting every tile's
      // reads, which would run out of registers).
      f16x4 P[NTILE];
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
      // An opaque 1.0 keeps fma(f16 -> f32, 1, acc) as one v_fma_mix_f32
      // instead of a conversion plus an add.
      float one = 1.0f;
      asm volatile("" : "+v"(one));
      constexpr int NB = 4;  // key-fragment buffers: reads run two steps ahead of use
      bf16x8 bkb[NB][KF];
      bf16x8 tbk[2];  // packed tail blocks of two groups of four tiles
      // The lane's byte offset is made opaque once per row block so the
      // compiler does not keep one address register per tile live.
      int lofs = lane * 16;
      asm volatile("" : "+v"(lofs));
      // Lanes whose dims lie beyond D read the next tile's data or the zero
      // pad: finite values whose query partners in A are zero.  The packed
      // tail block of group t/4 is read with tile 4 (t/4).
      auto lds_b = [&](int t, bf16x8 (&bk)[KF]) {
#pragma unroll
        for (int s = 0; s < KF; ++s) bk[s] = *reinterpret_cast<const bf16x8*>(sK + lofs + frag_at(t, s));
        if (TP && t % 4 == 0)
          tbk[(t / 4) % 2] = *reinterpret_cast<const bf16x8*>(sK + lofs + tail_at(t / 4));
      };
      auto mm = [&](const bf16x8 (&bk)[KF], int t) {
        f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KF; ++s) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], bk[s], a, 0, 0, 0);
        if (TP) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(at[t % 4], tbk[(t / 4) % 2], a, 0, 0, 0);
        return a;
      };
#pragma unroll
      for (int t = 0; t < NB - 1; ++t)
        if (t < NTILE) lds_b(t, bkb[t]);
      f32x4 acc = mm(bkb[0], 0);
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        if (t + NB - 1 < NTILE) lds_b(t + NB - 1, bkb[(t + NB - 1) % NB]);
        f32x4 accn = acc;
        if (t + 1 < NTILE) accn = mm(bkb[(t + 1) % NB], t + 1);
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = fast_exp2(fmaf(acc[r], c2, -b[r]));
        if (t == NTILE - 1) {  // the last tile may hold columns >= N
#pragma unroll
          for (int r = 0; r < 4; ++r) p[r] = 16 * t + li < N ? p[r] : 0.f;
        }
        P[t] = pack_f16x4(p[0], p[1], p[2], p[3]);
        // Row sums of the rounded values the column MFMA will see, so every
        // normalised row sums to 1 up to fp32 rounding (v_fma_mix_f32).
#pragma unroll
        for (int r = 0; r < 4; ++r) rs[r] = fmaf((float)P[t][r], one, rs[r]);
        acc = accn;
        __builtin_amdgcn_sched_barrier(0);
      }
      // Row weights w = 1/l, split into an fp16 high part (A row 0) and the
      // fp16 residual (A row 1) over the 16 rows of the block.
      f16x4 wa;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float l = row16_sum(rs[r]);
        const int row = rb * 16 + 4 * lg + r;
        const float w = row < N ? __builtin_amdgcn_rcpf(l) : 0.f;
        const _Float16 hi = (_Float16)w;
        const _Float16 lo = (_Float16)(w - (float)hi);
        wa[r] = li == 0 ? hi : (li == 1 ? lo : (_Float16)0.f);
      }
      // Column sums: C[0][j] + C[1][j] sit in lanes 0-15 (registers 0 and 1);
      // lanes 16-63 hold rows 4..15 of C, exactly zero (A rows >= 2 are zero).
      // They accumulate in registers across the wave's row blocks (LDS float
      // atomics serialise per lane and would stall the whole CU).
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x16f16(wa, P[t], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        colacc[t] += c[0] + c[1];
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) af[s] = an[s];
    }
    if (lane < 16) {
#pragma unroll
      for (int t = 0; t < NTILE; ++t) myacc[16 * t + li] = colacc[t];
    }
    __syncthreads();
    const bool bad = ctl[1] != 0u;
    for (int j = tid; j < N; j += NT) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kRowWaves; ++w) sum += cacc[w * NC + j];
      if (!bad) colsum[(int64_t)item * N + j] = sum;
    }
    if (tid == 0) redo[item] = bad ? 1 : 0;
  }
}

// sal[f][j] = (1 / (H*N)) * sum_h colsum[f][h][j]; workgroup x covers
// columns 256 (x % bpf) .. of frame x / bpf (a 1-D grid: any frame count).
__global__ __launch_bounds__(256) void salience_mean_kernel(const float* __restrict__ colsum,
                                                           int H, int N, int bpf, float inv,
                                                           float* __restrict__ sal) {
  const int f = blockIdx.x / bpf;
  const int j = (blockIdx.x % bpf) * blockDim.x + threadIdx.x;
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

static int pick_tpw_colstat(int N) {
  const int per = ((N + 15) / 16 + kColWaves - 1) / kColWaves;
  const int opts[] = {1, 2, 3, 4, 6};
  for (int o : opts)
    if (o >= per) return o;
  return -1;
}

static size_t colstat_lds_bytes(int tpw, int D) {
  const int ncp = kColWaves * tpw * 16;
  return (size_t)ncp * D * 2 + (size_t)2 * kRowBlocks * 16 * 2 * kColWaves * 4 + (size_t)ncp * 4 +
         32;
}

template <int D, int TPW>
static hipError_t colstat_go(const void* q, const void* k, int FH, int N, float c2, float* colsum,
                             const int32_t* only, hipStream_t st) {
  const size_t lds = colstat_lds_bytes(TPW, D);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)salience_colstat_kernel<D, TPW>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, kSalMaxLds);
    (void)hipGetLastError();
    attr_set = true;
  }
  int grid = device_cu_count();
  if (grid > FH) grid = FH;
  hipLaunchKernelGGL((salience_colstat_kernel<D, TPW>), dim3(grid), dim3(kColWaves * kWave), lds, st,
                     (const bf16_t*)q, (const bf16_t*)k, FH, N, c2, colsum, only);
  return hipGetLastError();
}

template <int D>
static hipError_t colstat_tpw(int tpw, const void* q, const void* k, int FH, int N, float c2,
                              float* colsum, const int32_t* only, hipStream_t st) {
  switch (tpw) {
    case 1: return colstat_go<D, 1>(q, k, FH, N, c2, colsum, only, st);
    case 2: return colstat_go<D, 2>(q, k, FH, N, c2, colsum, only, st);
    case 3: return colstat_go<D, 3>(q, k, FH, N, c2, colsum, only, st);
    case 4: return colstat_go<D, 4>(q, k, FH, N, c2, colsum, only, st);
    case 6: return colstat_go<D, 6>(q, k, FH, N, c2, colsum, only, st);
    default: return hipErrorInvalidValue;
  }
}

// The column-stationary kernel covers D in {64, 72, 80, 96} when its LDS fits.
static bool colstat_ok(int N, int D) {
  if (D != 64 && D != 72 && D != 80 && D != 96) return false;
  const int tpw = pick_tpw_colstat(N);
  return tpw > 0 && colstat_lds_bytes(tpw, D) <= (size_t)kSalMaxLds;
}

static hipError_t colstat_any(const void* q, const void* k, int FH, int N, int D, float c2,
                              float* colsum, const int32_t* only, hipStream_t st) {
  const int tpw = pick_tpw_colstat(N);
  switch (D) {
    case 64: return colstat_tpw<64>(tpw, q, k, FH, N, c2, colsum, only, st);
    case 72: return colstat_tpw<72>(tpw, q, k, FH, N, c2, colsum, only, st);
    case 80: return colstat_tpw<80>(tpw, q, k, FH, N, c2, colsum, only, st);
    default: return colstat_tpw<96>(tpw, q, k, FH, N, c2, colsum, only, st);
  }
}

// Row-stationary kernel: compiled for an exact number of 16-key column tiles,
// the square patch grids of common vision encoders: 13 (N in 193..208, e.g.
// 14 x 14 = 196), 16 (241..256), 25 (385..400, 20 x 20), 36 (561..576,
// 24 x 24) and 46 (721..736, 27 x 27 = 729).
static int pick_ntm_rows(int N) {
  const int nt = (N + 15) / 16;
  return (nt == 13 || nt == 16 || nt == 25 || nt == 36 || nt == 46) ? nt : -1;
}

static size_t rows_lds_bytes(int ntm, int D) {
  return (size_t)rows_k_bytes(D, ntm) + (size_t)kRowWaves * ntm * 16 * 4 + 16;
}

static bool rows_ok(int N, int D) {
  if (D != 64 && D != 72 && D != 80 && D != 96) return false;
  const int ntm = pick_ntm_rows(N);
  return ntm > 0 && rows_lds_bytes(ntm, D) <= (size_t)kSalMaxLds && colstat_ok(N, D);
}

template <int D, int NTM>
static hipError_t rows_go(const void* q, const void* k, int FH, int N, float c2, float* colsum,
                          int32_t* redo, hipStream_t st) {
  int grid = device_cu_count();
  if (grid > FH) grid = FH;
  const size_t lds = rows_lds_bytes(NTM, D);
  if (lds > (size_t)kSalMaxLds) return hipErrorInvalidValue;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)salience_rows_kernel<D, NTM>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, kSalMaxLds);
    (void)hipGetLastError();
    attr_set = true;
  }
  hipLaunchKernelGGL((salience_rows_kernel<D, NTM>), dim3(grid), dim3(kRowWaves * kWave), lds, st,
                     (const bf16_t*)q, (const bf16_t*)k, FH, N, c2, colsum, redo);
  return hipGetLastError();
}

template <int D>
static hipError_t rows_ntm(const void* q, const void* k, int FH, int N, float c2, float* colsum,
                           int32_t* redo, hipStream_t st) {
  switch (pick_ntm_rows(N)) {
    case 13: return rows_go<D, 13>(q, k, FH, N, c2, colsum, redo, st);
    case 16: return rows_go<D, 16>(q, k, FH, N, c2, colsum, redo, st);
    case 25: return rows_go<D, 25>(q, k, FH, N, c2, colsum, redo, st);
    case 36: return rows_go<D, 36>(q, k, FH, N, c2, colsum, redo, st);
    case 46: return rows_go<D, 46>(q, k, FH, N, c2, colsum, redo, st);
    default: return hipErrorInvalidValue;
  }
}

// The on-chip kernels (one frame-head's keys in LDS): N <= 768, D <= 96.
static bool onchip_ok(int N, int D) {
  if (N < 1 || D < 8 || D > 96 || D % 8) return false;
  const int tpw = pick_tpw(N);
  return tpw > 0 && sal_lds_bytes(tpw, D) <= (size_t)kSalMaxLds;
}

bool salience_supported(int N, int D) { return onchip_ok(N, D) || salience_stream_supported(N, D); }

hipError_t launch_salience(const void* q, const void* k, int F, int H, int N, int D, float scale,
                           float* colsum_ws, int32_t* redo_ws, float* lse_ws, float* sal,
                           hipStream_t st) {
  const float c2 = scale * 1.4426950408889634f;
  const int FH = F * H;
  hipError_t e;
  if (!onchip_ok(N, D)) {
    // Long frames (or wide heads): two streaming passes, lse then column sums.
    e = launch_salience_stream(q, k, FH, N, D, c2, lse_ws, colsum_ws, st);
  } else if (rows_ok(N, D)) {
    // fp16-probability row kernel, then the fp32 kernel on the items it flagged.
    switch (D) {
      case 64: e = rows_ntm<64>(q, k, FH, N, c2, colsum_ws, redo_ws, st); break;
      case 72: e = rows_ntm<72>(q, k, FH, N, c2, colsum_ws, redo_ws, st); break;
      case 80: e = rows_ntm<80>(q, k, FH, N, c2, colsum_ws, redo_ws, st); break;
      default: e = rows_ntm<96>(q, k, FH, N, c2, colsum_ws, redo_ws, st); break;
    }
    if (e == hipSuccess) e = colstat_any(q, k, FH, N, D, c2, colsum_ws, redo_ws, st);
  } else if (colstat_ok(N, D)) {
    e = colstat_any(q, k, FH, N, D, c2, colsum_ws, nullptr, st);
  } else {
    switch (pick_tpw(N)) {
      case 4: e = sal_ks<4>(q, k, FH, N, D, c2, colsum_ws, st); break;
      case 8: e = sal_ks<8>(q, k, FH, N, D, c2, colsum_ws, st); break;
      case 12: e = sal_ks<12>(q, k, FH, N, D, c2, colsum_ws, st); break;
      case 16: e = sal_ks<16>(q, k, FH, N, D, c2, colsum_ws, st); break;
      case 23: e = sal_ks<23>(q, k, FH, N, D, c2, colsum_ws, st); break;
      case 24: e = sal_ks<24>(q, k, FH, N, D, c2, colsum_ws, st); break;
      default: return hipErrorInvalidValue;
    }
  }
  if (e != hipSuccess) return e;
  const int bpf = (N + 255) / 256;
  hipLaunchKernelGGL(salience_mean_kernel, dim3((unsigned)((int64_t)F * bpf)), dim3(256), 0, st,
                     colsum_ws, H, N, bpf, 1.0f / ((float)H * (float)N), sal);
  return hipGetLastError();
}

}  // namespace sv
