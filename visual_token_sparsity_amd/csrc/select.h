// Exact top-k of one row of fp32 values by one workgroup (internal header).
//
// Keys are order-preserving uint32 images of the values (float_key).  Four
// 8-bit radix passes find the k-th largest key T and how many keys equal to T
// must be taken (ties go to the lowest indices).  A stable compaction then
// writes every index with key > T plus the first `remaining` indices with
// key == T, in ascending index order.  No sort.
//
// Element layout: wave w owns the contiguous segment [w*SEG, (w+1)*SEG) of
// the row (SEG a multiple of 64); lane l of wave w reads elements
// w*SEG + 64*i + l, so every load is a coalesced 256-byte access and the
// compaction needs only per-wave ballots plus one exchange of wave totals.
// Rows with N <= NW*64*KPT keep their keys in registers for all passes;
// longer rows are re-read (from L2) on every pass.
#pragma once

#include "common.h"

namespace sv {

template <int NW>
struct SelectSmem {
  uint32_t hist[256];
  uint32_t wtot[NW];
  uint32_t wcnt[NW][2];
  uint32_t digit, above;
};

// Inclusive block scan of one value per thread (NW waves).
template <int NW>
__device__ __forceinline__ uint32_t block_scan_incl(uint32_t v, uint32_t* wtot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  if (lane == kWave - 1) wtot[wave] = v;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w < wave) before += wtot[w];
  __syncthreads();
  return v + before;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Top-k of vals[0..N) -> out[0..k), ascending.  Called by all NW*64 threads.
// Requires 1 <= k <= N.  Coherent: read vals with device-coherent loads (the
// values were written by other workgroups of the same kernel).
template <int NW, int KPT, bool Coherent>
__device__ __forceinline__ void block_topk(const float* vals, int N, int k, int32_t* __restrict__ out,
                           SelectSmem<NW>& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int seg = ((N + NW * kWave - 1) / (NW * kWave)) * kWave;  // per-wave segment
  const int chunks = seg / kWave;
  const int base = wave * seg + lane;
  const bool cached = chunks <= KPT;

  auto ld = [&](int e) -> float { return Coherent ? load_shared_dev(vals + e) : vals[e]; };
  uint32_t key[KPT];
  if (cached) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = base + i * kWave;
      key[i] = (i < chunks && e < N) ? float_key(ld(e)) : 0u;
    }
  }
  // Visit this thread's elements in index order: f(e, valid, key).
  // Uniform across the wave (chunks is uniform), so ballots inside f are safe.
  auto for_each = [&](auto&& f) {
    if (cached) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        if (i < chunks) {
          const int e = base + i * kWave;
          f(e, e < N, key[i]);
        }
      }
    } else {
      for (int i = 0; i < chunks; ++i) {
        const int e = base + i * kWave;
        f(e, e < N, e < N ? float_key(ld(e)) : 0u);
      }
    }
  };

  if (tid == 0) {
    sm.digit = 0;
    sm.above = 0;
  }
  uint32_t prefix = 0, mask = 0, remaining = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += NW * kWave) sm.hist[b] = 0;
    __syncthreads();
    for_each([&](int e, bool valid, uint32_t kk) {
      if (valid && (kk & mask) == prefix) atomicAdd(&sm.hist[(kk >> shift) & 255u], 1u);
    });
    __syncthreads();
    // Suffix counts over the bins, highest digit first.
    static_assert(NW * kWave >= 256, "one bin per thread");
    const uint32_t c = tid < 256 ? sm.hist[255 - tid] : 0u;
    const uint32_t incl = block_scan_incl<NW>(c, sm.wtot);
    if (tid < 256) {
      const uint32_t excl = incl - c;
      if (excl < remaining && incl >= remaining) {
        sm.digit = 255u - tid;
        sm.above = excl;
      }
    }
    __syncthreads();
    remaining -= sm.above;
    prefix |= sm.digit << shift;
    mask |= 255u << shift;
  }
  const uint32_t thr = prefix;

  // Pass A: per-wave counts of keys > thr and == thr.
  uint32_t ngt = 0, neq = 0;
  for_each([&](int e, bool valid, uint32_t kk) {
    ngt += __popcll(__ballot(valid && kk > thr));
    neq += __popcll(__ballot(valid && kk == thr));
  });
  if (lane == 0) {
    sm.wcnt[wave][0] = ngt;
    sm.wcnt[wave][1] = neq;
  }
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) {
      gt_before += sm.wcnt[w][0];
      eq_before += sm.wcnt[w][1];
    }
  }
  // Pass B: stable write in index order.
  const uint64_t lt = lanemask_lt();
  for_each([&](int e, bool valid, uint32_t kk) {
    const bool g = valid && kk > thr;
    const bool q = valid && kk == thr;
    const uint64_t gm = __ballot(g);
    const uint64_t qm = __ballot(q);
    const uint32_t my_eq = eq_before + __popcll(qm & lt);
    if (g || (q && my_eq < remaining)) {
      const uint32_t pos = gt_before + __popcll(gm & lt) + (my_eq < remaining ? my_eq : remaining);
      if (pos < (uint32_t)k) out[pos] = e;
    }
    gt_before += __popcll(gm);
    eq_before += __popcll(qm);
  });
  __syncthreads();
}

}  // namespace sv
