// Sparse decode attention: the retrieved visual entries plus the text entries.
//
// SparseVILA velog summary, Sec. 3.2: only the query-relevant subset of the
// visual KV cache is activated for attention (the rest stays cached); Sec. 4.5
// (decoding attention kernel): decode is memory-bound, so the win comes from
// reading fewer KV bytes.
//
// Split-K flash-decode, one kernel.  Workgroup (c, g, b) takes entries
// [c*SE, (c+1)*SE) of the attended list E = idx[b][0..k) ++ text rows
// [0, txt_len[b]) and computes, for the G query heads of KV head g, a partial
// (m, l, acc) with the softmax in base 2 (the query is pre-scaled by
// scale*log2(e)).  Each lane group of LPE lanes owns EPL entries and reads
// their K and V head rows as 16-byte vectors straight from the cache (a
// gather: no packed copy is made), all loads in flight before any math.  With
// one split the workgroup normalises and writes the output; otherwise it
// publishes its partial with device-coherent stores, waits for them and bumps
// a counter for (b, g); the last workgroup reads the C partials with
// device-coherent loads, merges them by max-rescaling, writes the output and
// resets the counter to zero.
#include "common.h"

namespace sv {

constexpr int kAttnWaves = 4;

template <typename T, int D, int G, int EPL>
__global__ __launch_bounds__(kAttnWaves* kWave) void attn_kernel(
    const T* __restrict__ q, int Hq, const T* __restrict__ kv, const T* __restrict__ vv,
    int64_t vbs, int64_t vts, int N, const int32_t* __restrict__ idx, int k,
    const T* __restrict__ kt, const T* __restrict__ vt, int64_t tbs, int64_t tts,
    const int32_t* __restrict__ txt_len, int Tmax, float qscale, int C,
    float* __restrict__ part, uint32_t* __restrict__ counters, float* __restrict__ out) {
  constexpr int VE = Vec<T>::kElems;
  constexpr int LPE = D / VE;        // lanes per entry row of one head
  constexpr int EPW = kWave / LPE;   // entries per wave per step
  constexpr int SE = kAttnWaves * EPW * EPL;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int eg = lane / LPE, sub = lane % LPE, d0 = sub * VE;

  int tl = txt_len ? txt_len[b] : 0;
  tl = tl < 0 ? 0 : (tl > Tmax ? Tmax : tl);
  const int E = k + tl;
  const int e_begin = c * SE;

  // Entry -> cache row.  Visual indices outside [0, N) are skipped.
  int tok[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = e_begin + (j * kAttnWaves + wave) * EPW + eg;
    tok[j] = -1;
    if (e < k) tok[j] = idx[(int64_t)b * k + e];
  }
  Vec<T> qx[G];
#pragma unroll
  for (int i = 0; i < G; ++i) qx[i].load(q + ((int64_t)b * Hq + g * G + i) * D + d0);

  Vec<T> kx[EPL], vx[EPL];
  bool ok[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = e_begin + (j * kAttnWaves + wave) * EPW + eg;
    const T* kp = nullptr;
    const T* vp = nullptr;
    if (e < k) {
      const int t = tok[j];
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
    ok[j] = kp != nullptr;
    if (ok[j]) {
      kx[j].load(kp);
      vx[j].load(vp);
    } else {
      kx[j].zero();
      vx[j].zero();
    }
  }

  float qv[G][VE];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    qx[i].to_f32(qv[i]);
#pragma unroll
    for (int v = 0; v < VE; ++v) qv[i][v] *= qscale;
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
  for (int j = 0; j < EPL; ++j) {
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
  __shared__ uint32_t s_last;
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
  const int64_t head0 = (int64_t)b * Hq + g * G;
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
    if (C == 1) {
      out[(head0 + i) * D + d] = ll > 0.f ? aa / ll : 0.f;
    } else {
      float* pp = part + ((head0 + i) * C + c) * (D + 2);
      store_shared_dev(pp + d, aa);
      if (d == 0) {
        store_shared_dev(pp + D, mm);
        store_shared_dev(pp + D + 1, ll);
      }
    }
  }
  if (C == 1) return;

  wait_stores_complete();
  __syncthreads();
  uint32_t* ctr = counters + (int64_t)b * gridDim.y + g;
  if (threadIdx.x == 0) s_last = counter_add(ctr, 1u) == (uint32_t)C - 1 ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;

  // out = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c
  for (int t = threadIdx.x; t < G * D; t += kAttnWaves * kWave) {
    const int i = t / D, d = t % D;
    const float* pp = part + (head0 + i) * C * (D + 2);
    float M = -INFINITY;
#pragma unroll 8
    for (int cc = 0; cc < C; ++cc) M = fmaxf(M, load_shared_dev(pp + cc * (D + 2) + D));
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll 8
      for (int cc = 0; cc < C; ++cc) {
        const float mc = load_shared_dev(pp + cc * (D + 2) + D);
        const float f = (mc == -INFINITY) ? 0.f : fast_exp2(mc - M);
        num = fmaf(f, load_shared_dev(pp + cc * (D + 2) + d), num);
        den = fmaf(f, load_shared_dev(pp + cc * (D + 2) + D + 1), den);
      }
    }
    out[(head0 + i) * D + d] = den > 0.f ? num / den : 0.f;
  }
  if (threadIdx.x == 0) counter_reset(ctr);
}

static int entries_per_step(int D, int dtype) {
  const int VE = dtype == 1 ? 8 : 4;
  return kAttnWaves * (kWave / (D / VE));
}

int attn_splits(int B, int Hkv, int D, int dtype, int k, int Tmax, int* epl_out) {
  const int Emax = k + Tmax > 0 ? k + Tmax : 1;
  const int step = entries_per_step(D, dtype);
  // Most entries per lane (fewest partials, deepest load queue) that still
  // gives about four workgroups per CU.
  int epl = 8;
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

template <typename T, int D, int G, int EPL>
static hipError_t attn_go(const void* q, int B, int Hq, const void* kv, const void* vv, int64_t vbs,
                          int64_t vts, int N, int Hkv, const int32_t* idx, int k, const void* kt,
                          const void* vt, int64_t tbs, int64_t tts, const int32_t* txt_len,
                          int Tmax, float qscale, int C, float* out, float* part, uint32_t* ctr,
                          hipStream_t st) {
  hipLaunchKernelGGL((attn_kernel<T, D, G, EPL>), dim3(C, Hkv, B), dim3(kAttnWaves * kWave), 0, st,
                     (const T*)q, Hq, (const T*)kv, (const T*)vv, vbs, vts, N, idx, k, (const T*)kt,
                     (const T*)vt, tbs, tts, txt_len, Tmax, qscale, C, part, ctr, out);
  return hipGetLastError();
}

template <typename T, int D, int G>
static hipError_t attn_epl(int epl, const void* q, int B, int Hq, const void* kv, const void* vv,
                           int64_t vbs, int64_t vts, int N, int Hkv, const int32_t* idx, int k,
                           const void* kt, const void* vt, int64_t tbs, int64_t tts,
                           const int32_t* txt_len, int Tmax, float qs, int C, float* out,
                           float* part, uint32_t* ctr, hipStream_t st) {
#define SV_EPL_CASE(E)                                                                          \
  case E:                                                                                       \
    return attn_go<T, D, G, E>(q, B, Hq, kv, vv, vbs, vts, N, Hkv, idx, k, kt, vt, tbs, tts,    \
                               txt_len, Tmax, qs, C, out, part, ctr, st);
  switch (epl) {
    SV_EPL_CASE(1)
    SV_EPL_CASE(2)
    SV_EPL_CASE(4)
    SV_EPL_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef SV_EPL_CASE
}

template <typename T, int D>
static hipError_t attn_g(int G, int epl, const void* q, int B, int Hq, const void* kv,
                         const void* vv, int64_t vbs, int64_t vts, int N, int Hkv,
                         const int32_t* idx, int k, const void* kt, const void* vt, int64_t tbs,
                         int64_t tts, const int32_t* txt_len, int Tmax, float qs, int C,
                         float* out, float* part, uint32_t* ctr, hipStream_t st) {
#define SV_ATTN_CASE(GG)                                                                        \
  case GG:                                                                                      \
    return attn_epl<T, D, GG>(epl, q, B, Hq, kv, vv, vbs, vts, N, Hkv, idx, k, kt, vt, tbs, tts, \
                              txt_len, Tmax, qs, C, out, part, ctr, st);
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
                       float* part, uint32_t* counters, hipStream_t st) {
  const int G = Hq / Hkv;
  int epl = 1;
  const int C = attn_splits(B, Hkv, D, dtype, k, Tmax, &epl);
  const float qs = scale * 1.4426950408889634f;  // log2(e): the softmax runs in base 2
  if (dtype == 1) {
    if (D == 128)
      return attn_g<bf16_t, 128>(G, epl, q, B, Hq, kv, vv, vbs, vts, N, Hkv, idx, k, kt, vt, tbs,
                                 tts, txt_len, Tmax, qs, C, out, part, counters, st);
    return attn_g<bf16_t, 64>(G, epl, q, B, Hq, kv, vv, vbs, vts, N, Hkv, idx, k, kt, vt, tbs, tts,
                              txt_len, Tmax, qs, C, out, part, counters, st);
  }
  if (D == 128)
    return attn_g<float, 128>(G, epl, q, B, Hq, kv, vv, vbs, vts, N, Hkv, idx, k, kt, vt, tbs, tts,
                              txt_len, Tmax, qs, C, out, part, counters, st);
  return attn_g<float, 64>(G, epl, q, B, Hq, kv, vv, vbs, vts, N, Hkv, idx, k, kt, vt, tbs, tts,
                           txt_len, Tmax, qs, C, out, part, counters, st);
}

}  // namespace sv
