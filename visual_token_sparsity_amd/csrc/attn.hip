// Sparse decode attention: the retrieved visual entries plus the text entries.
//
// SparseVILA velog summary, Sec. 3.2: only the query-relevant subset of the
// visual KV cache is activated for attention (the rest stays cached); Sec. 4.5
// (decoding attention kernel): decode is memory-bound, so the win comes from
// reading fewer KV bytes.
//
// Split-K flash-decode.  Workgroup (c, g, b) takes entries [c*SE, (c+1)*SE) of
// the attended list E = idx[b][0..k) ++ text rows [0, txt_len[b]) and computes,
// for the G query heads of KV head g, a partial (m, l, acc) with an online
// softmax in base 2 (the query is pre-scaled by scale*log2(e)).  Each lane
// group of LPE lanes owns one entry at a time and reads its K and V head rows
// as 16-byte vectors straight from the cache (a gather: no packed copy is
// made), so each selected row is read once per KV head.  The combine kernel
// merges the C partials of each (b, h) by max-rescaling.
#include "common.h"

namespace sv {

constexpr int kAttnWaves = 4;
constexpr int kAttnEplMax = 4;  // entries per lane group per workgroup

template <typename T, int D, int G>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_partial_kernel(
    const T* __restrict__ q, int Hq, const T* __restrict__ kv, const T* __restrict__ vv,
    int64_t vbs, int64_t vts, int N, const int32_t* __restrict__ idx, int k,
    const T* __restrict__ kt, const T* __restrict__ vt, int64_t tbs, int64_t tts,
    const int32_t* __restrict__ txt_len, int Tmax, float qscale, int epl, int C,
    float* __restrict__ part) {
  constexpr int VE = Vec<T>::kElems;
  constexpr int LPE = D / VE;        // lanes per entry row of one head
  constexpr int EPW = kWave / LPE;   // entries per wave per step
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int eg = lane / LPE, sub = lane % LPE, d0 = sub * VE;

  int tl = txt_len ? txt_len[b] : 0;
  tl = tl < 0 ? 0 : (tl > Tmax ? Tmax : tl);
  const int E = k + tl;
  const int SE = kAttnWaves * EPW * epl;
  const int e_begin = c * SE;

  float qv[G][VE];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    Vec<T> x;
    x.load(q + ((int64_t)b * Hq + g * G + i) * D + d0);
    x.to_f32(qv[i]);
#pragma unroll
    for (int v = 0; v < VE; ++v) qv[i][v] *= qscale;
  }

  // Issue every load of this lane group's entries first (K and V vectors).
  Vec<T> kx[kAttnEplMax], vx[kAttnEplMax];
  bool ok[kAttnEplMax];
#pragma unroll
  for (int j = 0; j < kAttnEplMax; ++j) {
    ok[j] = false;
    kx[j].zero();
    vx[j].zero();
    if (j < epl) {
      const int e = e_begin + (j * kAttnWaves + wave) * EPW + eg;
      const T* kp = nullptr;
      const T* vp = nullptr;
      if (e < k) {
        const int t = idx[(int64_t)b * k + e];
        if (t >= 0 && t < N) {
          const int64_t off = (int64_t)b * vbs + (int64_t)t * vts + (int64_t)g * D + d0;
          kp = kv + off;
          vp = vv + off;
        }
      } else if (e < E) {
        const int64_t off = (int64_t)b * tbs + (int64_t)(e - k) * tts + (int64_t)g * D + d0;
        kp = kt + off;
        vp = vt + off;
      }
      if (kp) {
        ok[j] = true;
        kx[j].load(kp);
        vx[j].load(vp);
      }
    }
  }

  float m[G], l[G], acc[G][VE];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int v = 0; v < VE; ++v) acc[i][v] = 0.f;
  }

#pragma unroll
  for (int j = 0; j < kAttnEplMax; ++j) {
    if (j < epl) {
      float kf[VE], vf[VE];
      kx[j].to_f32(kf);
      vx[j].to_f32(vf);
      float z[G];
#pragma unroll
      for (int i = 0; i < G; ++i) {
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < VE; ++v) s = fmaf(qv[i][v], kf[v], s);
        z[i] = group_sum<LPE>(s);
      }
      if (ok[j]) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const float mn = fmaxf(m[i], z[i]);
          const float a = fast_exp2(m[i] - mn);  // m = -inf -> 0
          const float p = fast_exp2(z[i] - mn);
          l[i] = l[i] * a + p;
#pragma unroll
          for (int v = 0; v < VE; ++v) acc[i][v] = fmaf(p, vf[v], acc[i][v] * a);
          m[i] = mn;
        }
      }
    }
  }

  // Merge the EPW lane groups of this wave.
#pragma unroll
  for (int off = LPE; off < kWave; off <<= 1) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float mo = __shfl_xor(m[i], off, kWave);
      const float lo = __shfl_xor(l[i], off, kWave);
      const float mn = fmaxf(m[i], mo);
      const float a = (m[i] == -INFINITY) ? 0.f : fast_exp2(m[i] - mn);
      const float bo = (mo == -INFINITY) ? 0.f : fast_exp2(mo - mn);
      l[i] = l[i] * a + lo * bo;
#pragma unroll
      for (int v = 0; v < VE; ++v) {
        const float ao = __shfl_xor(acc[i][v], off, kWave);
        acc[i][v] = acc[i][v] * a + ao * bo;
      }
      m[i] = mn;
    }
  }

  // Merge the waves through LDS.
  __shared__ float s_ml[kAttnWaves][G][2];
  __shared__ float s_acc[kAttnWaves][G][D];
  if (eg == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
#pragma unroll
      for (int v = 0; v < VE; ++v) s_acc[wave][i][d0 + v] = acc[i][v];
      if (sub == 0) {
        s_ml[wave][i][0] = m[i];
        s_ml[wave][i][1] = l[i];
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G * D; t += kAttnWaves * kWave) {
    const int i = t / D, d = t % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) mm = fmaxf(mm, s_ml[w][i][0]);
    float ll = 0.f, aa = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float mw = s_ml[w][i][0];
      const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - mm);
      ll += s_ml[w][i][1] * f;
      aa += s_acc[w][i][d] * f;
    }
    float* pp = part + (((int64_t)b * Hq + g * G + i) * C + c) * (D + 2);
    pp[d] = aa;
    if (d == 0) {
      pp[D] = mm;
      pp[D + 1] = ll;
    }
  }
}

// out[b,h,d] = sum_c 2^(m_c - M) acc_c[d] / sum_c 2^(m_c - M) l_c
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part, int C,
                                                           int D, float* __restrict__ out) {
  const int bh = blockIdx.x;
  const float* pp = part + (int64_t)bh * C * (D + 2);
  float M = -INFINITY;
  for (int c = 0; c < C; ++c) M = fmaxf(M, pp[c * (D + 2) + D]);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
      for (int c = 0; c < C; ++c) {
        const float mc = pp[c * (D + 2) + D];
        if (mc == -INFINITY) continue;
        const float f = fast_exp2(mc - M);
        num = fmaf(f, pp[c * (D + 2) + d], num);
        den = fmaf(f, pp[c * (D + 2) + D + 1], den);
      }
    }
    out[(int64_t)bh * D + d] = den > 0.f ? num / den : 0.f;
  }
}

static int entries_per_step(int D, int dtype) {
  const int VE = dtype == 1 ? 8 : 4;
  return kAttnWaves * (kWave / (D / VE));
}

int attn_splits(int B, int Hkv, int D, int dtype, int k, int Tmax, int* epl_out) {
  const int Emax = k + Tmax;
  const int step = entries_per_step(D, dtype);
  // Smallest split that still gives every CU a few workgroups.
  int epl = kAttnEplMax;
  while (epl > 1) {
    const int se = step * epl;
    const long wgs = (long)((Emax + se - 1) / se) * Hkv * B;
    if (wgs >= 1024) break;
    epl >>= 1;
  }
  if (epl_out) *epl_out = epl;
  const int se = step * epl;
  return (Emax + se - 1) / se;
}

template <typename T, int D, int G>
static hipError_t attn_go(const void* q, int B, int Hq, const void* kv, const void* vv, int64_t vbs,
                          int64_t vts, int N, int Hkv, const int32_t* idx, int k, const void* kt,
                          const void* vt, int64_t tbs, int64_t tts, const int32_t* txt_len,
                          int Tmax, int dtype, float qscale, float* out, float* part,
                          hipStream_t st) {
  int epl = 1;
  const int C = attn_splits(B, Hkv, D, dtype, k, Tmax, &epl);
  hipLaunchKernelGGL((attn_partial_kernel<T, D, G>), dim3(C, Hkv, B), dim3(kAttnWaves * kWave), 0,
                     st, (const T*)q, Hq, (const T*)kv, (const T*)vv, vbs, vts, N, idx, k,
                     (const T*)kt, (const T*)vt, tbs, tts, txt_len, Tmax, qscale, epl, C, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(B * Hq), dim3(D), 0, st, part, C, D, out);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t attn_g(int G, const void* q, int B, int Hq, const void* kv, const void* vv,
                         int64_t vbs, int64_t vts, int N, int Hkv, const int32_t* idx, int k,
                         const void* kt, const void* vt, int64_t tbs, int64_t tts,
                         const int32_t* txt_len, int Tmax, int dtype, float qs, float* out,
                         float* part, hipStream_t st) {
#define SV_ATTN_CASE(GG)                                                                        \
  case GG:                                                                                      \
    return attn_go<T, D, GG>(q, B, Hq, kv, vv, vbs, vts, N, Hkv, idx, k, kt, vt, tbs, tts,      \
                             txt_len, Tmax, dtype, qs, out, part, st);
  switch (G) {
    SV_ATTN_CASE(1)
    SV_ATTN_CASE(2)
    SV_ATTN_CASE(3)
    SV_ATTN_CASE(4)
    SV_ATTN_CASE(5)
    SV_ATTN_CASE(6)
    SV_ATTN_CASE(7)
    SV_ATTN_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef SV_ATTN_CASE
}

hipError_t launch_attn(const void* q, int B, int Hq, const void* kv, const void* vv, int64_t vbs,
                       int64_t vts, int N, int Hkv, int D, const int32_t* idx, int k,
                       const void* kt, const void* vt, int64_t tbs, int64_t tts,
                       const int32_t* txt_len, int Tmax, int dtype, float scale, float* out,
                       float* part, hipStream_t st) {
  const int G = Hq / Hkv;
  const float qs = scale * 1.4426950408889634f;  // log2(e): the softmax runs in base 2
  if (dtype == 1) {
    if (D == 128)
      return attn_g<bf16_t, 128>(G, q, B, Hq, kv, vv, vbs, vts, N, Hkv, idx, k, kt, vt, tbs, tts,
                                 txt_len, Tmax, dtype, qs, out, part, st);
    return attn_g<bf16_t, 64>(G, q, B, Hq, kv, vv, vbs, vts, N, Hkv, idx, k, kt, vt, tbs, tts,
                              txt_len, Tmax, dtype, qs, out, part, st);
  }
  if (D == 128)
    return attn_g<float, 128>(G, q, B, Hq, kv, vv, vbs, vts, N, Hkv, idx, k, kt, vt, tbs, tts,
                              txt_len, Tmax, dtype, qs, out, part, st);
  return attn_g<float, 64>(G, q, B, Hq, kv, vv, vbs, vts, N, Hkv, idx, k, kt, vt, tbs, tts,
                           txt_len, Tmax, dtype, qs, out, part, st);
}

}  // namespace sv
