// Sparse decode attention over the retrieved visual entries plus the text
// entries (SparseVILA velog summary, Sec. 3.2: only the query-relevant subset
// of the visual KV cache is activated; Sec. 4.5: decode is memory-bound, so
// the win comes from reading fewer KV bytes).
//
// Split-K flash-decode in one kernel: workgroup (c, g, b) runs attention item
// c of KV head g of sequence b (decode_items.h); the last split of (b, g) to
// finish merges the partials and writes the output.
#include "decode_items.h"

namespace sv {

template <typename T, int D, int G, int EPL>
__global__ __launch_bounds__(kItemThreads) void attn_items_kernel(AttnArgs a) {
  extern __shared__ __align__(16) char smem[];
  attn_item<T, D, G, EPL>(a, blockIdx.z, blockIdx.y, blockIdx.x, false, smem);
}

AttnPlan attn_plan(int B, int Hkv, int D, int VE, int k, int Tmax, long target_items) {
  // Most entries per lane (fewest partials, deepest load queue) that still
  // gives about target_items workgroups.  When even one entry per lane does
  // not (few sequences and KV heads, long lists), keep the split count per
  // (sequence, KV head) at most kMaxSplits instead: the combine reads every
  // split, and many tiny splits cost more than they overlap.
  constexpr int kMaxSplits = 32;
  auto plan = [&](int epl) {
    AttnPlan p{};
    p.EPL = epl;
    p.SE = attn_split_entries(VE, D, epl);
    p.CT = (Tmax + p.SE - 1) / p.SE;
    p.CV = (k + p.SE - 1) / p.SE;
    return p;
  };
  for (int epl = 8; epl >= 1; epl >>= 1) {
    const AttnPlan p = plan(epl);
    if ((long)(p.CT + p.CV) * Hkv * B >= target_items) return p;
  }
  for (int epl = 1; epl < 8; epl <<= 1) {
    const AttnPlan p = plan(epl);
    if (p.CT + p.CV <= kMaxSplits) return p;
  }
  return plan(8);
}

AttnPlan fused_attn_plan(int B, int Hkv, int D, int VE, int k, int Tmax, int N) {
  AttnPlan p = attn_plan(B, Hkv, D, VE, k, Tmax, kFusedAttnTargetItems);
  if (p.EPL < 4) {
    p.EPL = 4;
    p.SE = attn_split_entries(VE, D, 4);
    p.CT = (Tmax + p.SE - 1) / p.SE;
    p.CV = (k + p.SE - 1) / p.SE;
  }
  // Chunk attention: one visual split per 2048-score chunk, whatever its
  // count of selected tokens (SE per round).
  if (fused_chunk_attn(B, Hkv, N, k)) p.CV = (N + 2047) / 2048;
  return p;
}

template <typename T, int D, int G, int EPL>
static hipError_t attn_go(const AttnArgs& a, int B, hipStream_t st) {
  const dim3 grid(a.CT + a.CV, a.Hkv, B);
  const size_t lds = attn_smem_bytes<D, G>();
  hipLaunchKernelGGL((attn_items_kernel<T, D, G, EPL>), grid, dim3(kItemThreads), lds, st, a);
  return hipGetLastError();
}

template <typename T, int D, int G>
static hipError_t attn_epl(int epl, const AttnArgs& a, int B, hipStream_t st) {
  switch (epl) {
    case 1: return attn_go<T, D, G, 1>(a, B, st);
    case 2: return attn_go<T, D, G, 2>(a, B, st);
    case 4: return attn_go<T, D, G, 4>(a, B, st);
    case 8: return attn_go<T, D, G, 8>(a, B, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D>
static hipError_t attn_g(int G, int epl, const AttnArgs& a, int B, hipStream_t st) {
  switch (G) {
    case 1: return attn_epl<T, D, 1>(epl, a, B, st);
    case 2: return attn_epl<T, D, 2>(epl, a, B, st);
    case 3: return attn_epl<T, D, 3>(epl, a, B, st);
    case 4: return attn_epl<T, D, 4>(epl, a, B, st);
    case 5: return attn_epl<T, D, 5>(epl, a, B, st);
    case 6: return attn_epl<T, D, 6>(epl, a, B, st);
    case 7: return attn_epl<T, D, 7>(epl, a, B, st);
    case 8: return attn_epl<T, D, 8>(epl, a, B, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn(const void* q, int B, int Hq, const void* kv, const void* vv, int64_t vbs,
                       int64_t vts, int N, int Hkv, int D, const int32_t* idx, int k,
                       const void* kt, const void* vt, int64_t tbs, int64_t tts,
                       const int32_t* txt_len, int Tmax, int dtype, float scale, float* out,
                       float* part, uint32_t* counters, int epl, hipStream_t st) {
  const int VE = dtype == 1 ? 8 : 4;
  AttnPlan p = attn_plan(B, Hkv, D, VE, k, Tmax, kAttnTargetItems);
  if (epl > 0) {
    p.EPL = epl;
    p.SE = attn_split_entries(VE, D, epl);
    p.CT = (Tmax + p.SE - 1) / p.SE;
    p.CV = (k + p.SE - 1) / p.SE;
  }
  AttnArgs a{};
  a.q = q;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.kv = kv;
  a.vv = vv;
  a.vbs = vbs;
  a.vts = vts;
  a.N = N;
  a.idx = idx;
  a.k = k;
  a.kt = kt;
  a.vt = vt;
  a.tbs = tbs;
  a.tts = tts;
  a.txt_len = txt_len;
  a.Tmax = Tmax;
  a.qscale = scale * 1.4426950408889634f;  // log2(e): the softmax runs in base 2
  a.CT = p.CT;
  a.CV = p.CV;
  a.part = part;
  a.comb_ctr = counters;
  a.out = out;
  a.ready = nullptr;
  const int G = Hq / Hkv;
  if (dtype == 1)
    return D == 128 ? attn_g<bf16_t, 128>(G, p.EPL, a, B, st) : attn_g<bf16_t, 64>(G, p.EPL, a, B, st);
  return D == 128 ? attn_g<float, 128>(G, p.EPL, a, B, st) : attn_g<float, 64>(G, p.EPL, a, B, st);
}

}  // namespace sv
