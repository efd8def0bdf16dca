// Exact top-k of long score rows, spread over many workgroups of the fused
// decode layer (internal header).
//
// The selection rule is that of the single-workgroup select (select.h; the
// retrieval step of SparseVILA velog summary, Sec. 3.2): the k largest
// scores of the row, equal scores taken toward the lower token index, the
// indices written in ascending order.  A row of N scores with N above one
// workgroup's registers would otherwise be read pass after pass by one
// workgroup, each read a round trip to memory; here every pass over the row
// is split into 2048-score chunks:
//
//   scan items   every score's top 11 key bits (digit d1) go to a local LDS
//                histogram, flushed with atomics to one of 8 replicas of a
//                per-sequence histogram (hist1); then one of the 16 count
//                lines of b += 1 (kLsScanCtrs: one hot line would serialise).
//   cand item p  (one per chunk, waits for all scan items of b) sums the
//                replicas, finds the digit D1 holding the k-th key, counts
//                its chunk's keys above D1 (chunk_hi[p]), appends the keys
//                in D1 to a per-sequence candidate list (one atomic per wave)
//                and adds their next 11 bits (digit d2) to hist2.
//   thr item     (waits for all cand items) finds the digit D2 of hist2
//                holding the remaining rank, ranks the candidates in
//                (D1, D2) to get the threshold key T and the last index Ti
//                taken among keys equal to T, counts every chunk's selected
//                keys and writes each chunk's first output position.
//   compact p    (waits for the thr item) writes the indices of its chunk's
//                selected keys {key > T, or key == T and index <= Ti} in
//                order; the last one raises ready[b].
//
// If D1 holds more than kLsCandCap keys, or (D1, D2) more than kLsFinalCap,
// the thr item runs the single-workgroup select over the whole row instead
// and the compaction items only count.  Each XCD dispatches its share of
// the grid in increasing order and every item waits only on items of lower
// index, so all waits end; all are bounded as well.
#pragma once

#include "decode_items.h"

namespace sv {

constexpr int kLsChunk = 2048;     // scores per candidate / compaction item
constexpr int kLsCandCap = 16384;  // keys of digit D1 kept as candidates
constexpr int kLsFinalCap = 256;   // keys of (D1, D2) ranked by one workgroup
constexpr int kLsCtlLines = 6;     // control lines per sequence
constexpr int kLsScanCtrLog2 = 4;  // the scan items' count lines per sequence: 16
constexpr int kLsScanCtrs = 1 << kLsScanCtrLog2;

static_assert(kLsChunk == kItemThreads * kSelKpt, "one chunk: eight keys per thread");
static_assert(kLsFinalCap <= kItemThreads, "one final candidate per thread");

struct LongSelArgs {
  uint32_t* hist1;     // [B][kLsReps][kLsBins]
  uint32_t* hist2;     // [B][kLsBins]
  uint64_t* cand;      // [B][kLsCandCap] key | index << 32
  uint32_t* chunk_hi;  // [B][P] keys of chunk p in digits above D1
  uint32_t* offs;      // [B][P] first output position of chunk p
  // [B][kLsCtlLines] lines of kCtrStride words: cand_n, cand_done,
  // thr_ready (1: compact, 2: already selected), comp_done, info1 (D1,
  // keys above D1, keys in D1, and D1 + 1 published early for the chunk
  // attention items), info2 (T, Ti).
  uint32_t* ctl;
  int P;               // chunks per row
  // Items that read (thr_ready, T, Ti) of a sequence: the P compaction items,
  // plus the Hkv*P chunk attention items when the visual attention runs
  // chunk by chunk (chunk_attn).  The last of them clears those words.
  uint32_t readers;
  bool chunk_attn;
};

__device__ __forceinline__ uint32_t* ls_line(const LongSelArgs& l, int b, int i) {
  return l.ctl + ((int64_t)b * kLsCtlLines + i) * kCtrStride;
}
enum { kLsCandN = 0, kLsCandDone = 1, kLsThrReady = 2, kLsCompDone = 3, kLsInfo1 = 4, kLsInfo2 = 5 };

// Chunk attention: (T, Ti) as one 64-bit word, T | (Ti + 1) << 32 (zero: not
// published yet), in words 2-3 of the info2 line.
__device__ __forceinline__ uint64_t* thr_pub_word(const LongSelArgs& l, int b) {
  return reinterpret_cast<uint64_t*>(ls_line(l, b, kLsInfo2) + 2);
}

__device__ __forceinline__ uint32_t digit1(uint32_t key) { return key >> 21; }
__device__ __forceinline__ uint32_t digit2(uint32_t key) { return (key >> 10) & (kLsBins - 1); }

// Poll a counter line until it reaches `target` (thread 0 of the
// workgroup), at most `limit` times; a wait that gives up ORs `bit` into the
// status word.  Returns the last value read.
__device__ __forceinline__ uint32_t poll_until(const uint32_t* p, uint32_t target, uint32_t limit,
                                               uint32_t* status, uint32_t bit) {
  uint32_t v = 0;
  for (uint32_t n = 0; n < limit; ++n) {
    v = load_flag(p);
    if (v >= target) return v;
    __builtin_amdgcn_s_sleep(4);
  }
  report_giveup(status, bit);
  return v;
}

// The sum of the n (<= 64) counter lines at p (kCtrStride apart), polled by a
// whole wave until it reaches `target`, at most `limit` times; otherwise as
// poll_until.  Every lane returns the last sum read.
__device__ __forceinline__ uint32_t wave_poll_sum_until(const uint32_t* p, int n, uint32_t target,
                                                        uint32_t limit, uint32_t* status,
                                                        uint32_t bit) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t v = 0;
  for (uint32_t it = 0; it < limit; ++it) {
    // Counts stay far below 2^24, so the float sum is exact.
    const float c = lane < n ? (float)load_flag(p + lane * kCtrStride) : 0.f;
    v = (uint32_t)group_sum<kWave>(c);
    if (v >= target) return v;
    __builtin_amdgcn_s_sleep(4);
  }
  if (lane == 0) report_giveup(status, bit);
  return v;
}

// Keys of chunk p of row b, eight per thread: element
// p*kLsChunk + wave*512 + i*64 + lane (the select's layout: each wave a
// contiguous run, ordered compaction by ballots).  Past the row: key 0,
// valid false.
__device__ __forceinline__ void load_chunk_keys(const float* scores, int N, int b, int p,
                                                uint32_t (&key)[kSelKpt], int& e0) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_uniform(threadIdx.x / kWave);
  const int c0 = p * kLsChunk;
  const int n = min(kLsChunk, N - c0);
  const BufRsrc r = make_rsrc(scores + (int64_t)b * N + c0, (uint32_t)n * 4u);
  e0 = c0 + wave * (kLsChunk / kItemWaves) + lane;
  const uint32_t o = (uint32_t)(wave * (kLsChunk / kItemWaves) + lane) * 4u;
  uint32_t w[kSelKpt];
#pragma unroll
  for (int i = 0; i < kSelKpt; ++i) w[i] = load1_dev(r, o + (uint32_t)i * kWave * 4u);
#pragma unroll
  for (int i = 0; i < kSelKpt; ++i) key[i] = float_key(__uint_as_float(w[i]));
}

// ---------------------------------------------------------------- cand item
struct CandSmem {
  uint32_t h1[kSelHistWords];
  uint32_t h2[kLsBins];
  uint32_t whi[kItemWaves];
  uint32_t d1, above1, c1;
};

__device__ __forceinline__ void cand_item(const ScanArgs& a, const LongSelArgs& l, int b, int p,
                                          char* smem) {
  CandSmem& sm = *reinterpret_cast<CandSmem*>(smem);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_uniform(tid / kWave);
  for (int i = tid; i < kLsBins; i += kItemThreads) sm.h2[i] = 0;
  if (wave == 0)
    wave_poll_sum_until(&a.seq_ctr[(b << a.ctr_log2) * kCtrStride], 1 << a.ctr_log2,
                        (uint32_t)a.items_per_seq, a.spin_limit, a.status, kGiveUpScanCount);
  __syncthreads();

  uint32_t key[kSelKpt];
  int e0;
  load_chunk_keys(a.scores, a.N, b, p, key, e0);
  // Sum of the replicas: bins 4*tid.. and 1024 + 4*tid..
  const BufRsrc hr = make_rsrc(l.hist1 + (int64_t)b * kLsReps * kLsBins,
                               (uint32_t)(kLsReps * kLsBins * 4));
  u32x4 s0 = {0u, 0u, 0u, 0u}, s1 = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int r = 0; r < kLsReps; ++r) {
    s0 += load4_dev(hr, (uint32_t)((r * kLsBins + 4 * tid) * 4));
    s1 += load4_dev(hr, (uint32_t)((r * kLsBins + kLsBins / 2 + 4 * tid) * 4));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sm.h1[sel_bin((uint32_t)(4 * tid + j))] = s0[j];
    sm.h1[sel_bin((uint32_t)(kLsBins / 2 + 4 * tid + j))] = s1[j];
  }
  __syncthreads();
  if (wave == 0) wave_find_digit(sm.h1, kLsBins, (uint32_t)a.k, &sm.d1, &sm.above1, &sm.c1);
  __syncthreads();
  const uint32_t D1 = sm.d1, c1 = sm.c1;
  const bool keep = c1 <= (uint32_t)kLsCandCap;  // uniform
  // Keys above D1 are selected whatever the threshold: the chunk attention
  // items start on them now.
  if (l.chunk_attn && p == 0 && tid == 0) store_flag(ls_line(l, b, kLsInfo1) + 3, D1 + 1u);

  uint32_t hi = 0, nc = 0;
#pragma unroll
  for (int i = 0; i < kSelKpt; ++i) {
    const bool valid = e0 + i * kWave < a.N;
    const uint32_t d = digit1(key[i]);
    hi += (valid && d > D1) ? 1u : 0u;
    nc += (valid && d == D1) ? 1u : 0u;
  }
  if (keep) {
    // One atomic per wave reserves the wave's slots in the candidate list.
    const uint32_t incl = wave_incl_scan(nc);
    const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
    uint32_t base = 0;
    if (lane == 0 && wtot) base = counter_add(ls_line(l, b, kLsCandN), wtot);
    base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
    uint32_t slot = base + incl - nc;
    uint64_t* cl = l.cand + (int64_t)b * kLsCandCap;
#pragma unroll
    for (int i = 0; i < kSelKpt; ++i) {
      const int e = e0 + i * kWave;
      const bool valid = e < a.N;
      if (valid && digit1(key[i]) == D1) {
        if (slot < (uint32_t)kLsCandCap)
          __hip_atomic_store(cl + slot, (uint64_t)key[i] | ((uint64_t)(uint32_t)e << 32),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        atomicAdd(&sm.h2[digit2(key[i])], 1u);
        ++slot;
      }
    }
  }
  const uint32_t hincl = wave_incl_scan(hi);
  if (lane == kWave - 1) sm.whi[wave] = hincl;
  __syncthreads();
  if (keep) {
    uint32_t* g2 = l.hist2 + (int64_t)b * kLsBins;
    for (int i = tid; i < kLsBins; i += kItemThreads) {
      const uint32_t v = sm.h2[i];
      if (v) __hip_atomic_fetch_add(g2 + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (tid == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kItemWaves; ++w) t += sm.whi[w];
    store_flag(l.chunk_hi + (int64_t)b * l.P + p, t);
    if (p == 0) {
      uint32_t* info = ls_line(l, b, kLsInfo1);
      store_flag(info + 0, D1);
      store_flag(info + 1, sm.above1);
      store_flag(info + 2, c1);
    }
  }
  wait_stores_complete();
  __syncthreads();
  if (tid == 0) counter_add(ls_line(l, b, kLsCandDone), 1u);
}

// ---------------------------------------------------------------- thr item
struct ThrSmem {
  uint32_t h2[kSelHistWords];
  uint32_t fk[kLsFinalCap], fi[kLsFinalCap];  // keys and indices of (D1, D2)
  uint32_t wsum[kItemWaves];
  uint32_t d2, above2, c2, nfin, tkey, tidx;
  uint32_t cnt[1];  // [P] selected keys per chunk (dynamic LDS past the struct)
};

__host__ __device__ inline size_t thr_smem_bytes(int P) {
  return sizeof(ThrSmem) + (size_t)(P > 1 ? P - 1 : 0) * sizeof(uint32_t);
}
__host__ __device__ inline size_t cand_smem_bytes() { return sizeof(CandSmem); }

__device__ __forceinline__ void thr_item(const ScanArgs& a, const LongSelArgs& l, int b,
                                         char* smem) {
  ThrSmem& sm = *reinterpret_cast<ThrSmem*>(smem);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_uniform(tid / kWave);
  const int P = l.P;
  if (tid == 0) {
    poll_until(ls_line(l, b, kLsCandDone), (uint32_t)P, a.spin_limit, a.status, kGiveUpCandCount);
    sm.nfin = 0;
  }
  __syncthreads();
  __builtin_amdgcn_s_setprio(3);  // every later item of b waits on this one

  const uint32_t* info = ls_line(l, b, kLsInfo1);
  const uint32_t above1 = load_flag(info + 1), c1 = load_flag(info + 2);
  {
    const BufRsrc hr = make_rsrc(l.hist2 + (int64_t)b * kLsBins, (uint32_t)(kLsBins * 4));
    const u32x4 s0 = load4_dev(hr, (uint32_t)(4 * tid * 4));
    const u32x4 s1 = load4_dev(hr, (uint32_t)((kLsBins / 2 + 4 * tid) * 4));
    const uint32_t* ch = l.chunk_hi + (int64_t)b * P;
    for (int i = tid; i < P; i += kItemThreads) sm.cnt[i] = load_flag(ch + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sm.h2[sel_bin((uint32_t)(4 * tid + j))] = s0[j];
      sm.h2[sel_bin((uint32_t)(kLsBins / 2 + 4 * tid + j))] = s1[j];
    }
  }
  bool fallback = c1 > (uint32_t)kLsCandCap;  // uniform
  __syncthreads();
  if (!fallback) {
    const uint32_t rem1 = (uint32_t)a.k - above1;  // 1 <= rem1 <= c1
    if (wave == 0) wave_find_digit(sm.h2, kLsBins, rem1, &sm.d2, &sm.above2, &sm.c2);
    __syncthreads();
    const uint32_t D2 = sm.d2, c2 = sm.c2;
    fallback = c2 > (uint32_t)kLsFinalCap;
    if (!fallback) {
      // Candidates of D1: those above D2 are taken (counted per chunk for the
      // compaction offsets); those in D2 go to LDS.  With chunk attention the
      // counting waits until the threshold is published: the attention items
      // wait on the threshold, only the compaction items on the counts.
      const uint64_t* cl = l.cand + (int64_t)b * kLsCandCap;
      auto cand_pass = [&](bool count, bool collect) {
        for (uint32_t s0 = 0; s0 < c1; s0 += 8 * kItemThreads) {
          uint64_t c[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t s = s0 + (uint32_t)(j * kItemThreads + tid);
            c[j] = s < c1 ? __hip_atomic_load(cl + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t s = s0 + (uint32_t)(j * kItemThreads + tid);
            if (s < c1) {
              const uint32_t kk = (uint32_t)c[j], e = (uint32_t)(c[j] >> 32);
              const uint32_t d = digit2(kk);
              if (d > D2) {
                if (count) atomicAdd(&sm.cnt[min(e / kLsChunk, (uint32_t)P - 1)], 1u);
              } else if (d == D2 && collect) {
                const uint32_t f = atomicAdd(&sm.nfin, 1u);
                if (f < (uint32_t)kLsFinalCap) {
                  sm.fk[f] = kk;
                  sm.fi[f] = e;
                }
              }
            }
          }
        }
      };
      cand_pass(!l.chunk_attn, true);
      __syncthreads();
      // The rem2-th of (D1, D2) by (key descending, index ascending) is the threshold.
      const uint32_t rem2 = rem1 - sm.above2;  // 1 <= rem2 <= c2
      uint32_t mk = 0, mi = 0;
      bool mine = (uint32_t)tid < c2;
      if (mine) {
        mk = sm.fk[tid];
        mi = sm.fi[tid];
        uint32_t rank = 0;
        for (uint32_t j = 0; j < c2; ++j) {
          const uint32_t ok = sm.fk[j], oi = sm.fi[j];
          rank += (ok > mk || (ok == mk && oi < mi)) ? 1u : 0u;
        }
        if (rank == rem2 - 1) {
          sm.tkey = mk;
          sm.tidx = mi;
        }
      }
      __syncthreads();
      const uint32_t T = sm.tkey, Ti = sm.tidx;
      if (l.chunk_attn) {
        if (tid == 0)
          __hip_atomic_store(thr_pub_word(l, b), (uint64_t)T | ((uint64_t)(Ti + 1u) << 32),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        cand_pass(true, false);
      }
      if (mine && (mk > T || (mk == T && mi <= Ti)))
        atomicAdd(&sm.cnt[min(mi / kLsChunk, (uint32_t)P - 1)], 1u);
      __syncthreads();
      // Exclusive scan of the chunk counts: each thread a contiguous run.
      const int per = (P + kItemThreads - 1) / kItemThreads;
      const int i0 = tid * per;
      uint32_t run = 0;
      for (int i = i0; i < i0 + per && i < P; ++i) run += sm.cnt[i];
      const uint32_t incl = wave_incl_scan(run);
      if (lane == kWave - 1) sm.wsum[wave] = incl;
      __syncthreads();
      uint32_t pos = incl - run;
#pragma unroll
      for (int w = 0; w < kItemWaves; ++w)
        if (w < wave) pos += sm.wsum[w];
      uint32_t* of = l.offs + (int64_t)b * P;
      for (int i = i0; i < i0 + per && i < P; ++i) {
        store_flag(of + i, pos);
        pos += sm.cnt[i];
      }
      if (tid == 0) {
        uint32_t* info2 = ls_line(l, b, kLsInfo2);
        store_flag(info2 + 0, T);
        store_flag(info2 + 1, Ti);
      }
    }
  }
  if (fallback) {
    __syncthreads();  // the select reuses the LDS
    SelectSmem<kItemWaves>& ss = *reinterpret_cast<SelectSmem<kItemWaves>*>(smem);
    block_topk<kItemWaves, kSelKpt, true, false>(a.scores + (int64_t)b * a.N, a.N, a.k,
                                                 a.idx + (int64_t)b * a.k, ss, nullptr,
                                                 a.idx_enc ? a.idx_enc + (int64_t)b * a.k : nullptr,
                                                 l.chunk_attn ? thr_pub_word(l, b) : nullptr);
  }
  wait_stores_complete();
  __syncthreads();
  if (tid == 0) store_flag(ls_line(l, b, kLsThrReady), fallback ? 2u : 1u);
  __builtin_amdgcn_s_setprio(0);

  // Every cand item has finished: clear what they used for the next launch.
  const u32x4 z = {0u, 0u, 0u, 0u};
  const BufRsrc h1 = make_rsrc(l.hist1 + (int64_t)b * kLsReps * kLsBins,
                               (uint32_t)(kLsReps * kLsBins * 4));
  for (int i = tid; i < kLsReps * kLsBins / 4; i += kItemThreads) store4_dev(h1, (uint32_t)(i * 16), z);
  const BufRsrc h2 = make_rsrc(l.hist2 + (int64_t)b * kLsBins, (uint32_t)(kLsBins * 4));
  for (int i = tid; i < kLsBins / 4; i += kItemThreads) store4_dev(h2, (uint32_t)(i * 16), z);
  if (tid < 3) counter_reset(ls_line(l, b, kLsInfo1) + tid);
  if (tid < (1 << a.ctr_log2)) counter_reset(&a.seq_ctr[((b << a.ctr_log2) + tid) * kCtrStride]);
  if (tid == 0) {
    counter_reset(ls_line(l, b, kLsCandN));
    counter_reset(ls_line(l, b, kLsCandDone));
  }
}

// One reader of (thr_ready, T, Ti) of b is done with them (thread 0); the
// last of l.readers clears them, and the early D1, for the next launch, and
// returns true.
__device__ __forceinline__ bool threshold_read_done(const LongSelArgs& l, int b) {
  if (counter_add(ls_line(l, b, kLsCompDone), 1u) != l.readers - 1) return false;
  counter_reset(ls_line(l, b, kLsCompDone));
  counter_reset(ls_line(l, b, kLsThrReady));
  counter_reset(ls_line(l, b, kLsInfo2));
  counter_reset(ls_line(l, b, kLsInfo2) + 1);
  if (l.chunk_attn) {
    counter_reset(ls_line(l, b, kLsInfo1) + 3);
    __hip_atomic_store(thr_pub_word(l, b), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return true;
}

// ---------------------------------------------------------------- compact item
struct CompactSmem {
  uint32_t mode;
  uint32_t wcnt[kItemWaves];
};

__device__ __forceinline__ void compact_item(const ScanArgs& a, const LongSelArgs& l, int b, int p,
                                             char* smem) {
  CompactSmem& sm = *reinterpret_cast<CompactSmem*>(smem);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_uniform(tid / kWave);
  if (tid == 0)
    sm.mode = poll_until(ls_line(l, b, kLsThrReady), 1u, a.spin_limit, a.status, kGiveUpThreshold);
  __syncthreads();
  if (sm.mode == 1u) {
    uint32_t key[kSelKpt];
    int e0;
    load_chunk_keys(a.scores, a.N, b, p, key, e0);
    const uint32_t* info2 = ls_line(l, b, kLsInfo2);
    const uint32_t T = load_flag(info2 + 0), Ti = load_flag(info2 + 1);
    const uint32_t base = load_flag(l.offs + (int64_t)b * l.P + p);
    const int cend = min(a.N, p * kLsChunk + kLsChunk);
    bool sel[kSelKpt];
    uint32_t n = 0;
#pragma unroll
    for (int i = 0; i < kSelKpt; ++i) {
      const int e = e0 + i * kWave;
      sel[i] = e < cend && (key[i] > T || (key[i] == T && (uint32_t)e <= Ti));
      n += (uint32_t)__popcll(__ballot(sel[i]));
    }
    if (lane == 0) sm.wcnt[wave] = n;
    __syncthreads();
    uint32_t pos = base;
#pragma unroll
    for (int w = 0; w < kItemWaves; ++w)
      if (w < wave) pos += sm.wcnt[w];
    const uint64_t lt = lanemask_lt();
    int32_t* out = a.idx + (int64_t)b * a.k;
#pragma unroll
    for (int i = 0; i < kSelKpt; ++i) {
      const uint64_t bm = __ballot(sel[i]);
      const uint32_t o = pos + (uint32_t)__popcll(bm & lt);
      if (sel[i] && o < (uint32_t)a.k) {
        __hip_atomic_store(out + o, (int32_t)(e0 + i * kWave), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (a.idx_enc)
          __hip_atomic_store(a.idx_enc + (int64_t)b * a.k + o, (uint32_t)(e0 + i * kWave) + 1u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      pos += (uint32_t)__popcll(bm);
    }
  }
  wait_stores_complete();
  __syncthreads();
  if (tid == 0 && threshold_read_done(l, b) && a.ready) store_flag(&a.ready[b * kCtrStride], 1u);
}

// ---------------------------------------------------------------- chunk attention lists
// The selected tokens of chunk p of row b, for the attention item of (b, g, p)
// (every thread calls): first the keys above D1 (selected whatever the
// threshold), once D1 is published; then, through more(), the selected keys
// of digit D1 ({key > T, or key == T and index <= Ti}, the select's rule),
// once the threshold is.  Both lists are in ascending token order, written
// to list (LDS, kLsChunk entries); wcnt is kItemWaves + 2 words of LDS.
struct ChunkSel {
  uint32_t key[kSelKpt];
  int e0, cend;
  uint32_t D1;
};

// Appends to list[base ..] the chunk's keys above D1 (tail false) or its
// selected keys of digit D1 under the threshold (T, Ti) (tail true); returns
// the new length.
__device__ __forceinline__ int chunk_list_append(const ChunkSel& cs, int* list, uint32_t* wcnt,
                                                 int base, bool tail, uint32_t T, uint32_t Ti) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_uniform(tid / kWave);
  bool sel[kSelKpt];
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < kSelKpt; ++i) {
    const int e = cs.e0 + i * kWave;
    const uint32_t d = digit1(cs.key[i]);
    sel[i] = e < cs.cend &&
             (tail ? (d == cs.D1 && (cs.key[i] > T || (cs.key[i] == T && (uint32_t)e <= Ti)))
                   : d > cs.D1);
    n += (uint32_t)__popcll(__ballot(sel[i]));
  }
  if (lane == 0) wcnt[wave] = n;
  __syncthreads();
  int pos = base, total = 0;
#pragma unroll
  for (int w = 0; w < kItemWaves; ++w) {
    pos += w < wave ? (int)wcnt[w] : 0;
    total += (int)wcnt[w];
  }
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int i = 0; i < kSelKpt; ++i) {
    const uint64_t bm = __ballot(sel[i]);
    if (sel[i]) list[pos + __popcll(bm & lt)] = cs.e0 + i * kWave;
    pos += __popcll(bm);
  }
  __syncthreads();
  return base + total;
}

}  // namespace sv
