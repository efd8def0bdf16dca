// Exact top-k of one row of fp32 values by one workgroup (internal header).
//
// Order: value descending, ties to the lower index (keys are the
// order-preserving uint32 images of the values, float_key, so -0 == +0).
// The result is the k selected indices in ascending order.
//
// Fast path (no contended atomics).  The value range [min, max] is split
// into 2048 equal bins; the bin map is monotone in the value, so every key in
// a higher bin beats every key in a lower one.  A histogram (spread values
// put a handful of keys in each bin, so the LDS atomics rarely collide)
// gives the bin B that holds the k-th key and the count `above` of keys in
// higher bins.  The keys of bin B (at most 256 of them) are ranked exactly
// against each other; the one of rank k-above-1 is the threshold element
// (T_key, T_idx).  Element e is selected iff key_e > T_key, or key_e ==
// T_key and e <= T_idx: exactly k elements.
//
// Fallback (all values equal, non-finite range, or more than 256 keys in bin
// B): three exact radix passes (11, 11 and 10 bits) find the k-th key T and
// how many keys equal to T to take, lowest indices first.
//
// Either way a stable compaction writes the selected indices in ascending
// order: per-wave ballots plus one exchange of wave totals.  Element layout:
// wave w owns the contiguous segment [w*SEG, (w+1)*SEG) of the row (SEG a
// multiple of 64); lane l of wave w reads elements w*SEG + 64*i + l, so
// every load is a coalesced 256-byte access.  Rows with N <= NW*64*KPT keep
// their keys in registers; longer rows are re-read on every pass.
#pragma once

#include "common.h"

namespace sv {

// A value the same in every lane of the wave, kept in a scalar register.  A
// division by a kernel argument runs on the vector unit, and a buffer
// resource or loop bound built from its result would otherwise take a
// per-lane loop around every load that uses it.
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

constexpr int kSelBins = 2048;                        // widest digit: 11 bits
constexpr int kSelHistWords = kSelBins + kSelBins / 32;  // one pad word per 32 bins

constexpr int kSelMaxCand = 256;

template <int NW>
struct SelectSmem {
  uint32_t hist[2][kSelHistWords];  // fast path: hist[1] holds the candidates
  uint32_t wcnt[NW][2];
  float wmin[NW], wmax[NW];
  uint32_t digit, above, count, ncand;
  uint32_t thr_key, thr_idx;
};

__device__ __forceinline__ int sel_bin(uint32_t d) { return (int)(d + (d >> 5)); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// One wave: the digit of an nb-bin histogram h (LDS, padded layout
// sel_bin; highest digit first) that holds the `remaining`-th key.  The one
// lane that finds it writes (digit, keys in higher bins, keys in the
// digit's bin) to the three outputs (LDS).  Each lane sums its run of nb/64
// bins (independent reads), a DPP scan finds the run holding the crossing,
// and the wave scans that run one bin per lane.
__device__ __forceinline__ void wave_find_digit(const uint32_t* h, int nb, uint32_t remaining,
                                                uint32_t* digit, uint32_t* above,
                                                uint32_t* count) {
  const int lane = threadIdx.x & (kWave - 1);
  const int per = nb / kWave;
  const int hi = nb - 1 - lane * per;
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < kSelBins / kWave; ++j)
    if (j < per) tot += h[sel_bin((uint32_t)(hi - j))];
  const uint32_t incl = wave_incl_scan(tot);
  const uint32_t excl = incl - tot;
  const uint64_t hit = __ballot(excl < remaining && incl >= remaining);  // one lane
  const int hl = hit ? (int)__builtin_ctzll(hit) : 0;
  const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)excl, hl);
  const int top = nb - 1 - hl * per;
  const uint32_t c = lane < per ? h[sel_bin((uint32_t)(top - lane))] : 0u;
  const uint32_t ci = wave_incl_scan(c);
  if (lane < per && base + ci >= remaining && base + ci - c < remaining) {  // one lane
    *digit = (uint32_t)(top - lane);
    *above = base + ci - c;
    *count = c;
  }
}

// Top-k of vals[0..N) -> out[0..k), ascending.  Called by all NW*64 threads.
// Requires 1 <= k <= N.  Coherent: read vals with device-coherent loads (the
// values were written by other workgroups of the same kernel) and write out
// with device-coherent stores (other workgroups of the kernel read it).
// Cached: the row fits in registers (N <= NW*64*KPT); otherwise it is
// re-read on every pass.  pre: the caller already holds the keys of a cached
// row, in this layout; vals is then not read.  out == nullptr: compute
// everything, write nothing (runs the code once, e.g. to warm the
// instruction cache while waiting for the scores).  out_enc: also write
// each index plus one there (device-coherent; zero means not written).
// thr_pub: also publish the threshold element there as one device-coherent
// 64-bit word, T_key | (T_idx + 1) << 32 (never zero).
template <int NW, int KPT, bool Coherent, bool Cached>
__device__ __forceinline__ void block_topk(const float* vals, int N, int k, int32_t* __restrict__ out,
                           SelectSmem<NW>& sm, const uint32_t* pre = nullptr,
                           uint32_t* __restrict__ out_enc = nullptr,
                           uint64_t* __restrict__ thr_pub = nullptr) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_uniform(tid / kWave);
  const int seg = ((N + NW * kWave - 1) / (NW * kWave)) * kWave;  // per-wave segment
  const int chunks = seg / kWave;
  const int base = wave * seg + lane;
  constexpr bool cached = Cached;

  auto ld = [&](int e) -> float { return Coherent ? load_shared_dev(vals + e) : vals[e]; };
  uint32_t key[KPT];
  if constexpr (cached) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = base + i * kWave;
      key[i] = pre ? pre[i] : ((i < chunks && e < N) ? float_key(ld(e)) : 0u);
    }
  }
  // Visit this thread's elements in index order: f(e, valid, key).
  // Uniform across the wave (chunks is uniform), so ballots inside f are safe.
  auto for_each = [&](auto&& f) {
    if constexpr (cached) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        if (i < chunks) {
          const int e = base + i * kWave;
          f(e, e < N, key[i]);
        }
      }
    } else {
      // Batches of 8 loads in flight, then the visits in index order.
      for (int i0 = 0; i0 < chunks; i0 += 8) {
        uint32_t kb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int e = base + (i0 + j) * kWave;
          kb[j] = (i0 + j < chunks && e < N) ? float_key(ld(e)) : 0u;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (i0 + j < chunks) {
            const int e = base + (i0 + j) * kWave;
            f(e, e < N, kb[j]);
          }
        }
      }
    }
  };

  static_assert(NW >= 2, "wave 0 scans while the others clear");
  static_assert(NW * kWave >= kSelMaxCand, "one candidate per thread");

  // Wave 0: find the digit of an nb-bin histogram (highest first) holding
  // the `remaining`-th key; sets sm.digit, sm.above (keys in higher bins) and
  // sm.count (keys in the digit's bin).  Each lane sums its run of nb/64 bins
  // (independent reads), a lane scan finds the run that holds the crossing,
  // and the wave then scans that run one bin per lane.
  auto find_digit = [&](const uint32_t* h, int nb, uint32_t remaining) {
    wave_find_digit(h, nb, remaining, &sm.digit, &sm.above, &sm.count);
  };

  // ---- value range (and a cleared histogram)
  float vmin = INFINITY, vmax = -INFINITY;
  for_each([&](int e, bool valid, uint32_t kk) {
    if (valid) {
      const float v = key_to_float(kk);
      vmin = fminf(vmin, v);
      vmax = fmaxf(vmax, v);
    }
  });
  wave_minmax(vmin, vmax);
  if (lane == 0) {
    sm.wmin[wave] = vmin;
    sm.wmax[wave] = vmax;
  }
  for (int b = tid; b < kSelHistWords; b += NW * kWave) sm.hist[0][b] = 0;
  if (tid == 0) sm.ncand = 0;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    vmin = fminf(vmin, sm.wmin[w]);
    vmax = fmaxf(vmax, sm.wmax[w]);
  }
  const float scale = (float)kSelBins / (vmax - vmin);
  bool fast = vmax > vmin && scale > 0.f && scale < INFINITY;  // uniform

  // ---- binned histogram, the bin of the k-th key, its candidates
  uint32_t thr_key = 0, thr_idx = 0;
  if (fast) {
    auto bin_of = [&](uint32_t kk) -> uint32_t {
      const float x = (key_to_float(kk) - vmin) * scale;
      return (uint32_t)fminf(fmaxf(x, 0.f), (float)(kSelBins - 1));
    };
    for_each([&](int e, bool valid, uint32_t kk) {
      if (valid) atomicAdd(&sm.hist[0][sel_bin(bin_of(kk))], 1u);
    });
    __syncthreads();
    if (wave == 0) find_digit(sm.hist[0], kSelBins, (uint32_t)k);
    __syncthreads();
    const uint32_t bstar = sm.digit, above = sm.above, cnt = sm.count;
    fast = cnt <= (uint32_t)kSelMaxCand;  // uniform
    if (cnt == 1) {
      // The bin holds one key (the usual case for spread values): it is the
      // threshold element (k - above = 1), written by the thread that owns it;
      // no candidate list and no ranking.
      for_each([&](int e, bool valid, uint32_t kk) {
        if (valid && bin_of(kk) == bstar) {
          sm.thr_key = kk;
          sm.thr_idx = (uint32_t)e;
        }
      });
      __syncthreads();
      thr_key = sm.thr_key;
      thr_idx = sm.thr_idx;
    } else if (fast) {
      uint32_t* cand = sm.hist[1];  // [kSelMaxCand] keys, then [kSelMaxCand] indices
      for_each([&](int e, bool valid, uint32_t kk) {
        if (valid && bin_of(kk) == bstar) {
          // cnt <= kSelMaxCand keys fall in bin bstar; the bound only guards
          // against inconsistent inputs (a wait that gave up).
          const uint32_t slot = atomicAdd(&sm.ncand, 1u);
          if (slot < (uint32_t)kSelMaxCand) {
            cand[slot] = kk;
            cand[kSelMaxCand + slot] = (uint32_t)e;
          }
        }
      });
      __syncthreads();
      const uint32_t rem = (uint32_t)k - above;  // 1 <= rem <= cnt
      if ((uint32_t)tid < cnt) {
        const uint32_t mk = cand[tid], mi = cand[kSelMaxCand + tid];
        // Broadcast reads, eight candidates in flight per step.
        uint32_t rank = 0;
        for (uint32_t j0 = 0; j0 < cnt; j0 += 8) {
#pragma unroll
          for (uint32_t j = j0; j < j0 + 8; ++j) {
            const uint32_t ok = cand[j], oi = cand[kSelMaxCand + j];
            rank += (j < cnt && (ok > mk || (ok == mk && oi < mi))) ? 1u : 0u;
          }
        }
        if (rank == rem - 1) {
          sm.thr_key = mk;
          sm.thr_idx = mi;
        }
      }
      __syncthreads();
      thr_key = sm.thr_key;
      thr_idx = sm.thr_idx;
    }
  }

  if (!fast) {
    // ---- exact radix passes: the k-th key T and the number of ties to take
    for (int b = tid; b < kSelHistWords; b += NW * kWave) sm.hist[0][b] = 0;
    __syncthreads();
    uint32_t prefix = 0, mask = 0, remaining = (uint32_t)k;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const int shift = p == 0 ? 21 : (p == 1 ? 10 : 0);
      const int nb = p == 2 ? 1024 : 2048;
      uint32_t* h = sm.hist[p & 1];
      for_each([&](int e, bool valid, uint32_t kk) {
        if (valid && (kk & mask) == prefix) atomicAdd(&h[sel_bin((kk >> shift) & (uint32_t)(nb - 1))], 1u);
      });
      __syncthreads();
      if (wave == 0) {
        find_digit(h, nb, remaining);
      } else if (p < 2) {
        uint32_t* hn = sm.hist[(p + 1) & 1];
        for (int b = tid - kWave; b < kSelHistWords; b += (NW - 1) * kWave) hn[b] = 0;
      }
      __syncthreads();
      remaining -= sm.above;
      prefix |= sm.digit << shift;
      mask |= (uint32_t)(nb - 1) << shift;
    }
    // The remaining-th key equal to T (in index order) is the threshold element.
    thr_key = prefix;
    uint32_t neq = 0;
    for_each([&](int e, bool valid, uint32_t kk) { neq += __popcll(__ballot(valid && kk == prefix)); });
    if (lane == 0) sm.wcnt[wave][1] = neq;
    __syncthreads();
    uint32_t eq_before = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w < wave) eq_before += sm.wcnt[w][1];
    const uint64_t lt = lanemask_lt();
    for_each([&](int e, bool valid, uint32_t kk) {
      const bool q = valid && kk == prefix;
      const uint64_t qm = __ballot(q);
      if (q && eq_before + __popcll(qm & lt) == remaining - 1) sm.thr_idx = (uint32_t)e;
      eq_before += __popcll(qm);
    });
    __syncthreads();
    thr_idx = sm.thr_idx;
  }

  if (thr_pub && tid == 0)
    __hip_atomic_store(thr_pub, (uint64_t)thr_key | ((uint64_t)(thr_idx + 1u) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- stable compaction of {e : key_e > T_key or (key_e == T_key and e <= T_idx)}
  auto selected = [&](int e, bool valid, uint32_t kk) {
    return valid && (kk > thr_key || (kk == thr_key && (uint32_t)e <= thr_idx));
  };
  uint32_t nsel = 0;
  for_each([&](int e, bool valid, uint32_t kk) { nsel += __popcll(__ballot(selected(e, valid, kk))); });
  if (lane == 0) sm.wcnt[wave][0] = nsel;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w < wave) before += sm.wcnt[w][0];
  const uint64_t lt = lanemask_lt();
  for_each([&](int e, bool valid, uint32_t kk) {
    const bool sel = selected(e, valid, kk);
    const uint64_t bm = __ballot(sel);
    const uint32_t pos = before + __popcll(bm & lt);
    if (sel && pos < (uint32_t)k && out != nullptr) {
      if (Coherent)
        __hip_atomic_store(out + pos, (int32_t)e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        out[pos] = e;
      if (out_enc)
        __hip_atomic_store(out_enc + pos, (uint32_t)e + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    before += __popcll(bm);
  });
  __syncthreads();
}

}  // namespace sv
