// Work items of the decode hot path (internal header), shared by the
// standalone retrieval kernel, the standalone attention kernel and the fused
// per-layer kernel.
//
// Scan item (SparseVILA velog summary, Sec. 3.2, Query-Aware Token Selection;
// xllm-io review, core formulas): scores s[b,t] = sum_g qhat[b,g,:] . K[b,t,g,:]
// for a contiguous run of cache rows of sequence b, where qhat[b,g] is the sum
// of the query over its Tq tokens and the G query heads of KV head g.  The
// score is linear in the query, so summing first equals summing per-head
// logits.  qhat lives in LDS (two planes of four floats per 16-byte chunk, so
// a wave's reads are conflict-free); registers hold only two rows of keys in
// flight per lane.  A row of C 16-byte chunks is split into segments of at
// most 64*CPL chunks; LPR lanes (a power of two) cover one segment with up to
// CPL chunks each (CPL = 8; 4 in the bf16 short-row scans, which keeps the
// fused kernel's short-row mode at five waves per SIMD).  Chunks past the row end read a clamped in-row address and
// meet a zero in qhat, so every load is unconditional.
//
// Select (same passage): when the last scan item of a sequence finishes, its
// workgroup takes the exact top-k of the score row (select.h).
//
// Attention item (velog summary, Sec. 3.2 and Sec. 4.5): split c of KV head g
// of sequence b.  Splits [0, CT) cover the text entries, splits [CT, CT+CV)
// the selected visual entries, SE entries each.  A lane group of LPE lanes
// owns EPL entries and reads their K and V head rows as 16-byte vectors (a
// gather: no packed copy is made), all loads in flight before any math; the
// softmax runs in base 2 on a query pre-scaled by scale*log2(e).  Partials
// (m, l, acc) go out with device-coherent stores; the last split of (b, g) to
// arrive merges them by max-rescaling and writes the output.
//
// bf16 caches with G >= 2 query heads per KV head take matrix cores instead:
// a wave owns tiles of 16 entries; S^T = K Q^T (v_mfma_f32_16x16x32_bf16, the
// G query heads as columns of a 16-wide B operand; each lane loads 16-byte
// slices of one entry's K row straight into the A operand), an online softmax
// per head column, then O^T += V^T P^T (v_mfma_f32_16x16x16_bf16 with P^T as
// a bf16 high part plus the bf16 residual, so the product keeps fp32 accuracy;
// V^T comes from the tile's V rows staged in the wave's LDS buffer and read
// with ds_read_tr16_b64).  The same splits, partials and combine.
#pragma once

#include <type_traits>

#include "common.h"
#include "select.h"

namespace sv {

constexpr int kItemWaves = 4;
constexpr int kItemThreads = kItemWaves * kWave;
constexpr int kScanCpl = 8;        // 16-byte chunks per lane per segment (default)
constexpr int kScanCplShort = 4;   // bf16 short-row scans (fused and standalone): half the registers
// Chunks per lane per unit of the short-row scans of a dtype (1: bf16).
template <typename T>
__host__ __device__ constexpr int short_scan_cpl() { return sizeof(T) == 2 ? kScanCplShort : kScanCpl; }
__host__ inline int short_scan_cpl(int dtype) { return dtype == 1 ? kScanCplShort : kScanCpl; }
constexpr int kSelKpt = 8;         // keys per thread kept in registers by the select

// Bits of the sticky status word (the first word of a workspace whose kernels
// wait on each other): a bounded wait that gave up ORs in its bit and the item
// carries on with what it read, so the outputs of that launch are invalid.
enum : uint32_t {
  kGiveUpScores = 1u,      // select item: score row never complete
  kGiveUpIndices = 2u,     // visual attention item: selected indices never complete
  kGiveUpScanCount = 4u,   // long-row candidate item: scan items never all counted
  kGiveUpCandCount = 8u,   // long-row threshold item: candidate items never all counted
  kGiveUpThreshold = 16u,  // long-row compaction item: threshold never published
};

__device__ __forceinline__ void report_giveup(uint32_t* status, uint32_t bit) {
  if (status) __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kLsReps = 8;         // replicas of a long row's first-level key histogram
constexpr int kLsBins = 2048;      // 11-bit key digits

// ---------------------------------------------------------------- scan
struct ScanArgs {
  const void* q;
  int Tq, Hq, G;
  const void* kv;
  int64_t bstride, tstride;  // elements
  int N, D;
  int C;                     // 16-byte chunks per row
  int nseg, LPR;             // segments per row, lanes per segment
  int rows_per_item, items_per_seq;
  float* scores;             // [B][N]
  int k;
  int32_t* idx;              // [B][k]
  uint32_t* seq_ctr;         // [B << ctr_log2] (stride kCtrStride) finished scan items, self-resetting
  // Long rows: scan item j of b counts on line (b << ctr_log2) + j % (1 << ctr_log2),
  // and the waiting items sum the 1 << ctr_log2 lines of b.  Atomics on one
  // address serialise (about 12 ns each), so one line per sequence would hold
  // the last count back by several microseconds when hundreds of items
  // finish together.  0 elsewhere (one line: the last arriver is known).
  int ctr_log2;
  uint32_t* ready;           // [B] (stride kCtrStride) selection published (fused kernel only)
  // Fused kernel, rows that fit the select's registers: scores are stored as
  // the complement of their bits (a zero word: not written yet) and a select
  // item polls the row; no counters.
  bool encode;
  // Fused kernel, longer rows: [B][kLsReps][kLsBins] histogram of the
  // scores' top 11 key bits, which every scan item adds to (long_select.h).
  // Null otherwise.
  uint32_t* hist1;
  // Fused kernel: [B][k] the selected indices plus one (zero: not written
  // yet), which the attention items poll; zero again after the launch.
  uint32_t* idx_enc;
  uint32_t spin_limit;       // polls before a wait gives up (>= 1)
  uint32_t* status;          // sticky status word (give-up bits), may be null
};

// Chunks of qhat kept in LDS (zero past C).
// A segment is cpl * 64 chunks (each lane cpl of them).
__host__ __device__ inline int scan_padded_chunks(int nseg, int LPR, int cpl = kScanCpl) {
  return nseg > 1 ? nseg * cpl * kWave : LPR * cpl;
}

__host__ inline void scan_geometry(int C, int* nseg, int* LPR, int cpl = kScanCpl) {
  const int seg = cpl * kWave;
  if (C > seg) {
    *nseg = (C + seg - 1) / seg;
    *LPR = kWave;
    return;
  }
  *nseg = 1;
  const int need = (C + cpl - 1) / cpl;
  int l = 1;
  while (l < need) l <<= 1;
  *LPR = l;
}

__device__ __forceinline__ float sum_lanes_rt(float v, int width) {
  switch (width) {  // wave-uniform
    case 1: return v;
    case 2: return lane_group_sum<2>(v);
    case 4: return lane_group_sum<4>(v);
    case 8: return lane_group_sum<8>(v);
    case 16: return lane_group_sum<16>(v);
    case 32: return lane_group_sum<32>(v);
    default: return lane_group_sum<64>(v);
  }
}

// One scan item: rows [item*rows_per_item, ...) of sequence b.  Returns true
// in every thread of the workgroup that must run the select for b.  q_of is
// the sequence whose qhat LDS holds (-1: none); it is reused when it matches.
// PAIR: one-segment rows take their two units of keys together, each qhat
// read feeding both FMA chains (more registers, half the LDS reads and two
// independent chains; each chain adds in the same order, so the same bits).
template <typename T, int CPL = kScanCpl, bool PAIR = false>
__device__ __forceinline__ bool scan_item(const ScanArgs& a, int b, int item, char* smem,
                                          int& q_of) {
  constexpr int VE = Vec<T>::kElems;
  constexpr int NP = VE / 4;  // float4 planes of qhat
  constexpr int ES = (int)sizeof(T);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_uniform(tid / kWave);
  const int LPR = a.LPR, nseg = a.nseg;
  const int RPS = kWave / LPR;  // units per wave step
  const int sub = lane & (LPR - 1);
  const int rsub = lane / LPR;
  constexpr int SEG = CPL * kWave;  // chunks per segment
  constexpr int QB = PAIR ? 8 : 1;  // query rows loaded together for qhat (GQA groups)
  const int CP = scan_padded_chunks(nseg, LPR, CPL);
  float* qh = reinterpret_cast<float*>(smem);  // [NP][CP][4]

  const int r0 = item * a.rows_per_item;
  int r1 = r0 + a.rows_per_item;
  r1 = r1 < a.N ? r1 : a.N;
  const int nrows = r1 - r0;
  // One-segment rows: blocks of RPS rows go to the waves in turn, so the four
  // waves read one contiguous run together (one stream per item).  Longer
  // rows: each wave a contiguous run of whole rows (its units are the
  // segments of one row after another).
  int nunits, wr0 = 0;
  if (nseg == 1) {
    const int nblk = (nrows + RPS - 1) / RPS;
    nunits = nblk > wave ? ((nblk - wave + kItemWaves - 1) / kItemWaves) * RPS : 0;
  } else {
    const int wrows = (nrows + kItemWaves - 1) / kItemWaves;
    wr0 = wave * wrows;  // relative to r0
    int wn = nrows - wr0;
    wn = wn < 0 ? 0 : (wn > wrows ? wrows : wn);
    nunits = wn * nseg;
  }

  // The item's rows as one buffer: row r at byte (r - r0) * row_bytes.
  const uint32_t row_bytes = (uint32_t)(a.tstride * ES);
  const BufRsrc rs = make_rsrc(
      reinterpret_cast<const char*>(a.kv) + ((int64_t)b * a.bstride + (int64_t)r0 * a.tstride) * ES,
      (uint32_t)(nrows - 1) * row_bytes + (uint32_t)a.C * 16u);
  // Unit u of this wave: row unit_row(u) (relative to r0), segment u % nseg.
  // Units past the wave's run, or rows past the item, read past the extent
  // (zeros, no memory traffic).
  auto unit_seg = [&](int u) { return nseg == 1 ? 0 : u % nseg; };
  auto unit_row = [&](int u) {
    return nseg == 1 ? ((u / RPS) * kItemWaves + wave) * RPS + u % RPS : wr0 + u / nseg;
  };
  auto unit_off = [&](int u) -> uint32_t {
    const int row = unit_row(u);
    if (u >= nunits || row >= nrows) return kBufOob;
    return (uint32_t)row * row_bytes + (uint32_t)(unit_seg(u) * SEG + sub) * 16u;
  };
  // Chunk j of a unit is chunk sub + j*LPR of its segment; chunks past the
  // segment are not loaded (uniform) or, where a segment is ragged, zeroed.
  auto load_unit = [&](int u, Vec<T>* dst) {
    const int slen = min(SEG, a.C - unit_seg(u < nunits ? u : 0) * SEG);
    const uint32_t off = unit_off(u);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      if (j * LPR < slen)
        dst[j].template load_buf<kCacheStream>(rs, off, (uint32_t)(j * LPR * 16));
      else
        dst[j].zero();
    }
  };
  auto mask_ragged = [&](int u, Vec<T>* v) {
    const int slen = min(SEG, a.C - unit_seg(u) * SEG);
    if (slen % LPR == 0) return;  // uniform
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      if (sub + j * LPR >= slen) v[j].zero();
  };

  // The wave's first two units of keys in flight before the query is summed
  // (units past the wave's run read nothing).
  Vec<T> va[CPL], vb[CPL];
  load_unit(rsub, va);
  load_unit(RPS + rsub, vb);

  // Long rows: a local histogram of the item's score digits, past qhat.
  uint32_t* lh = reinterpret_cast<uint32_t*>(smem + (size_t)CP * VE * sizeof(float));
  if (a.hist1) {
    for (int i = tid; i < kLsBins; i += kItemThreads) lh[i] = 0u;
    if (q_of == b) __syncthreads();  // otherwise the qhat barrier orders it
  }

  // qhat -> LDS (zero past C).
  if (q_of != b) {
    const T* qb = reinterpret_cast<const T*>(a.q);
    for (int c = tid; c < CP; c += kItemThreads) {
      float acc[VE];
#pragma unroll
      for (int v = 0; v < VE; ++v) acc[v] = 0.f;
      if (c < a.C) {
        const int e0 = c * VE;
        const int g = e0 / a.D, d0 = e0 % a.D;
        // Query row j = tau G + i of head group g, summed in row order.
        const int nq = a.Tq * a.G;
        const T* q0 = qb + ((int64_t)b * a.Tq * a.Hq + g * a.G) * a.D + d0;
        if constexpr (QB == 1) {
          for (int tau = 0; tau < a.Tq; ++tau)
            for (int i = 0; i < a.G; ++i) {
              Vec<T> x;
              x.load(q0 + ((int64_t)tau * a.Hq + i) * a.D);
              float f[VE];
              x.to_f32(f);
#pragma unroll
              for (int v = 0; v < VE; ++v) acc[v] += f[v];
            }
        } else {
          // QB loads in flight (past the last row: the last row again, not added).
          for (int j0 = 0; j0 < nq; j0 += QB) {
            Vec<T> x[QB];
#pragma unroll
            for (int jj = 0; jj < QB; ++jj) {
              const int j = j0 + jj < nq ? j0 + jj : nq - 1;
              const int tau = j / a.G, i = j - tau * a.G;
              x[jj].load(q0 + ((int64_t)tau * a.Hq + i) * a.D);
            }
#pragma unroll
            for (int jj = 0; jj < QB; ++jj) {
              if (j0 + jj < nq) {
                float f[VE];
                x[jj].to_f32(f);
#pragma unroll
                for (int v = 0; v < VE; ++v) acc[v] += f[v];
              }
            }
          }
        }
      }
#pragma unroll
      for (int p = 0; p < NP; ++p)
        *reinterpret_cast<f32x4v*>(qh + ((int64_t)p * CP + c) * 4) =
            f32x4v{acc[4 * p], acc[4 * p + 1], acc[4 * p + 2], acc[4 * p + 3]};
    }
    __syncthreads();
    q_of = b;
  }

  const bool coherent = a.k > 0;
  float* srow = a.scores + (int64_t)b * a.N + r0;
  float acc = 0.f;
  // The reduced score s of unit u's row (lanes with sub == 0 store it).
  auto store_score = [&](float s, int u) {
    const int row = unit_row(u);
    if (sub == 0 && u < nunits && row < nrows) {
      if (a.encode)
        __hip_atomic_store(reinterpret_cast<uint32_t*>(srow) + row, ~__float_as_uint(s),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else if (coherent) {
        store_shared_dev(srow + row, s);  // read back by the selecting workgroup
        if (a.hist1) atomicAdd(&lh[float_key(s) >> 21], 1u);
      } else
        srow[row] = s;
    }
  };
  // Unit u (keys in cur): the lanes' partial dot products, reduced and stored
  // at the row's last segment.
  auto consume = [&](Vec<T>* cur, int u) {
    const int seg = unit_seg(u);
    mask_ragged(u, cur);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int ch = seg * SEG + sub + j * LPR;
      float f[VE];
      cur[j].to_f32(f);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const f32x4v w = *reinterpret_cast<const f32x4v*>(qh + ((int64_t)p * CP + ch) * 4);
        acc = fmaf(w.x, f[4 * p], acc);
        acc = fmaf(w.y, f[4 * p + 1], acc);
        acc = fmaf(w.z, f[4 * p + 2], acc);
        acc = fmaf(w.w, f[4 * p + 3], acc);
      }
    }
    if (seg == nseg - 1) {
      store_score(sum_lanes_rt(acc, LPR), u);
      acc = 0.f;
    }
  };
  auto consume2 = [&](Vec<T>* ca, int ua, Vec<T>* cb, int ub) {
    mask_ragged(ua, ca);
    mask_ragged(ub, cb);
    float xa = 0.f, xb = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int ch = sub + j * LPR;
      float fa[VE], fb[VE];
      ca[j].to_f32(fa);
      cb[j].to_f32(fb);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const f32x4v w = *reinterpret_cast<const f32x4v*>(qh + ((int64_t)p * CP + ch) * 4);
        xa = fmaf(w.x, fa[4 * p], xa);
        xb = fmaf(w.x, fb[4 * p], xb);
        xa = fmaf(w.y, fa[4 * p + 1], xa);
        xb = fmaf(w.y, fb[4 * p + 1], xb);
        xa = fmaf(w.z, fa[4 * p + 2], xa);
        xb = fmaf(w.z, fb[4 * p + 2], xb);
        xa = fmaf(w.w, fa[4 * p + 3], xa);
        xb = fmaf(w.w, fb[4 * p + 3], xb);
      }
    }
    store_score(sum_lanes_rt(xa, LPR), ua);
    store_score(sum_lanes_rt(xb, LPR), ub);
  };
  // Two buffers, each refilled right after it is consumed, so two units per
  // lane stay in flight (steps are wave-uniform).
  if (PAIR && nseg == 1) {
    int u0 = 0;
    for (; u0 + RPS < nunits; u0 += 2 * RPS) {
      consume2(va, u0 + rsub, vb, u0 + RPS + rsub);
      if (u0 + 2 * RPS < nunits) load_unit(u0 + 2 * RPS + rsub, va);
      if (u0 + 3 * RPS < nunits) load_unit(u0 + 3 * RPS + rsub, vb);
    }
    if (u0 < nunits) consume(va, u0 + rsub);
  } else {
    for (int u0 = 0; u0 < nunits; u0 += 2 * RPS) {
      consume(va, u0 + rsub);
      if (u0 + 2 * RPS < nunits) load_unit(u0 + 2 * RPS + rsub, va);
      if (u0 + RPS < nunits) {
        consume(vb, u0 + RPS + rsub);
        if (u0 + 3 * RPS < nunits) load_unit(u0 + 3 * RPS + rsub, vb);
      }
    }
  }

  if (!coherent || a.encode) return false;
  __shared__ uint32_t s_last;
  if (a.hist1) {
    __syncthreads();
    uint32_t* g = a.hist1 + ((int64_t)b * kLsReps + (item & (kLsReps - 1))) * kLsBins;
    for (int i = tid; i < kLsBins; i += kItemThreads) {
      const uint32_t v = lh[i];
      if (v) __hip_atomic_fetch_add(g + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_stores_complete();
    __syncthreads();
    if (tid == 0) {
      const int line = (b << a.ctr_log2) + (item & ((1 << a.ctr_log2) - 1));
      counter_add(&a.seq_ctr[line * kCtrStride], 1u);
    }
    return false;
  }
  wait_stores_complete();
  __syncthreads();
  if (tid == 0)
    s_last = counter_add(&a.seq_ctr[b * kCtrStride], 1u) == (uint32_t)a.items_per_seq - 1 ? 1u : 0u;
  __syncthreads();
  return s_last != 0;
}

// Exact top-k of the score row of b into idx[b]; leaves idx visible to other
// workgroups of the kernel (device-coherent stores, completed) and resets the
// sequence counter.
__device__ __forceinline__ void select_item(const ScanArgs& a, int b, char* smem, int& q_of) {
  q_of = -1;  // the select overwrites qhat
  // Everything waiting on this sequence waits on this workgroup: let its
  // waves issue ahead of the streaming waves that share the CU.
  __builtin_amdgcn_s_setprio(3);
  SelectSmem<kItemWaves>& sm = *reinterpret_cast<SelectSmem<kItemWaves>*>(smem);
  const float* srow = a.scores + (int64_t)b * a.N;
  if (a.N <= kItemThreads * kSelKpt)
    block_topk<kItemWaves, kSelKpt, true, true>(srow, a.N, a.k, a.idx + (int64_t)b * a.k, sm);
  else
    block_topk<kItemWaves, kSelKpt, true, false>(srow, a.N, a.k, a.idx + (int64_t)b * a.k, sm);
  wait_stores_complete();
  __syncthreads();
  if (threadIdx.x == 0) {
    counter_reset(&a.seq_ctr[b * kCtrStride]);
    if (a.ready) store_flag(&a.ready[b * kCtrStride], 1u);
  }
  __builtin_amdgcn_s_setprio(0);
}

// Select item of the fused kernel (rows of at most kItemThreads*kSelKpt
// scores, stored complemented by the scan items): polls the score row of b
// until every word is written (completion detection and loading the keys
// are one and the same read), selects the top-k into idx[b], raises
// ready[b], then restores the words to zero for the next launch and
// optionally writes the decoded scores.
__device__ __forceinline__ void select_poll_item(const ScanArgs& a, int b, float* scores_out,
                                                 char* smem) {
  constexpr int NW = kItemWaves, KPT = kSelKpt;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_uniform(tid / kWave);
  const int N = a.N;
  const int seg = ((N + NW * kWave - 1) / (NW * kWave)) * kWave;
  const int chunks = seg / kWave;
  const int base = wave * seg + lane;
  uint32_t* words = reinterpret_cast<uint32_t*>(a.scores) + (int64_t)b * N;
  uint32_t w[KPT];
  for (uint32_t n = 0;; ++n) {
    bool missing = false;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = base + i * kWave;
      w[i] = (i < chunks && e < N)
                 ? __hip_atomic_load(words + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                 : 1u;
      missing |= w[i] == 0u;
    }
    if (!__syncthreads_or(missing)) break;
    if (n + 1 >= a.spin_limit) {
      if (tid == 0) report_giveup(a.status, kGiveUpScores);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  __builtin_amdgcn_s_setprio(3);
#pragma unroll
  for (int i = 0; i < KPT; ++i) w[i] = float_key(__uint_as_float(~w[i]));
  SelectSmem<NW>& sm = *reinterpret_cast<SelectSmem<NW>*>(smem);
  block_topk<NW, KPT, true, true>(nullptr, N, a.k, a.idx + (int64_t)b * a.k, sm, w,
                                  a.idx_enc ? a.idx_enc + (int64_t)b * a.k : nullptr);
  wait_stores_complete();
  __syncthreads();
  if (tid == 0) store_flag(&a.ready[b * kCtrStride], 1u);
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int e = base + i * kWave;
    if (i < chunks && e < N) {
      words[e] = 0u;  // ready for the next launch
      if (scores_out) scores_out[(int64_t)b * N + e] = key_to_float(w[i]);
    }
  }
}

__host__ __device__ inline size_t scan_smem_bytes(int nseg, int LPR, int VE, bool hist = false,
                                                  int cpl = kScanCpl) {
  const size_t q = (size_t)scan_padded_chunks(nseg, LPR, cpl) * VE * sizeof(float) +
                   (hist ? (size_t)kLsBins * sizeof(uint32_t) : 0);
  const size_t s = sizeof(SelectSmem<kItemWaves>);
  return q > s ? q : s;
}

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const void* q;
  int Hq, Hkv;
  const void* kv;
  const void* vv;
  int64_t vbs, vts;
  int N;
  const int32_t* idx;
  int k;
  const void* kt;
  const void* vt;
  int64_t tbs, tts;
  const int32_t* txt_len;
  int Tmax;
  float qscale;          // scale * log2(e)
  int CT, CV;            // text and visual splits
  float* part;           // [B][Hq][CT+CV][attn_part_stride(D)]
  uint32_t* comb_ctr;    // [B][Hkv] (stride kCtrStride), self-resetting
  float* out;            // [B][Hq][D]
  uint32_t* ready;       // [B] (stride kCtrStride; fused kernel only)
  uint32_t* vis_done;    // [B] (stride kCtrStride) finished visual items (fused kernel only)
  const uint32_t* idx_enc;  // [B][k] selected indices plus one, polled (fused kernel only)
  uint32_t spin_limit;      // polls before a wait gives up (>= 1)
  uint32_t* status;         // sticky status word (give-up bits), may be null
};

template <typename T, int D>
struct AttnShape {
  static constexpr int VE = Vec<T>::kElems;
  static constexpr int LPE = D / VE;       // lanes per entry row of one head
  static constexpr int EPW = kWave / LPE;  // entries per wave per step
};

// LDS of an attention item: the per-wave (acc, m, l) slots, reused by the
// combine for the weights and l of up to kMaxCombineSplits splits per head,
// G denominators and one float4 per thread.
constexpr int kMaxCombineSplits = 256;
constexpr int kAttnVPad = 32;  // bytes of padding per V row in the MFMA item's LDS buffer
template <int D>
__host__ __device__ constexpr size_t attn_mfma_vbuf_bytes() {
  return (size_t)16 * (2 * D + kAttnVPad);  // one 16-entry tile of V rows (bf16)
}
template <int D, int G>
__host__ __device__ constexpr size_t attn_smem_bytes() {
  const size_t w = (size_t)kItemWaves * G * (D + 2);
  const size_t c = (size_t)G * kMaxCombineSplits * 2 + 8 + (size_t)kItemThreads * 4;
  const size_t f = (w > c ? w : c) * sizeof(float);
  const size_t v = G >= 2 ? kItemWaves * attn_mfma_vbuf_bytes<D>() : 0;  // bf16 matrix-core item
  return f > v ? f : v;
}

// Float4 columns of the combine and the number of thread groups that split
// the splits among them (a power of two, at most 16).
template <int D, int G>
__host__ __device__ constexpr int combine_groups() {
  constexpr int V = G * D / 4;
  int s = 1;
  while (s < 16 && 2 * s * V <= kItemThreads) s *= 2;
  return s;
}

typedef __attribute__((ext_vector_type(8))) __bf16 attn_bf16x8;
typedef __attribute__((ext_vector_type(4))) float attn_f32x4;
typedef short attn_s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t attn_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Matrix-core front of a bf16 item with G >= 2 (see the header): entries
// [e0, e0 + n_ent) of the split, SE of them at most; writes each wave's
// (acc, m, l) per head into its LDS slot slot(w, i) = smem + (w*G + i)*(D+2)
// floats, as the vector front does.  LIST: the entries are the visual tokens
// list[0 .. n) (LDS), taken SE at a time with the softmax state carried from
// round to round; n starts at n_ent, and once those are done more() (called
// by every thread) may append entries and returns the new n, once.
template <int D, int G, int SE, bool LIST, class More>
__device__ __forceinline__ void attn_front_mfma(const AttnArgs& a, int b, int g, bool text,
                                                int e0, int n_ent, bool wait, char* smem,
                                                const int* list, More&& more) {
  static_assert(G >= 2 && G <= 16, "query heads as the columns of one 16-wide tile");
  constexpr int KS = D / 32, DB = D / 16;
  constexpr int TPW = (SE + 16 * kItemWaves - 1) / (16 * kItemWaves);  // tiles per wave
  constexpr int VSTR = 2 * D + kAttnVPad;
  constexpr int VCH = D / 8;               // 16-byte chunks per V row
  constexpr int VLD = 16 * VCH / kWave;    // V loads per lane per tile
  constexpr int VEPL = kWave / VCH;        // entries per V load instruction
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = wave_uniform(tid / kWave);
  const int li = lane & 15, lg = lane >> 4;
  const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q);

  // Q^T (B operand): lane (li, lg) holds head g*G + li (zero past G), dims
  // 32 s + 8 lg.
  attn_bf16x8 qf[KS];
  {
    const bf16_t* qh = q + ((int64_t)b * a.Hq + g * G + (li < G ? li : 0)) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 u = li < G ? *reinterpret_cast<const uint4*>(qh + 32 * s) : make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(attn_bf16x8, u);
    }
  }

  // The sequence's cache as one buffer (as in the vector front).
  const int64_t ts = text ? a.tts : a.vts;
  BufRsrc krs, vrs;
  {
    const int64_t rows = text ? (a.Tmax > 0 ? a.Tmax : 1) : (a.N > 0 ? a.N : 1);
    const uint32_t ext = (uint32_t)(((int64_t)(rows - 1) * ts + (int64_t)a.Hkv * D) * 2);
    const char* kb = reinterpret_cast<const char*>(text ? a.kt : a.kv) + (int64_t)b * (text ? a.tbs : a.vbs) * 2;
    const char* vb = reinterpret_cast<const char*>(text ? a.vt : a.vv) + (int64_t)b * (text ? a.tbs : a.vbs) * 2;
    krs = make_rsrc(kb, ext);
    vrs = make_rsrc(vb, ext);
  }
  const uint32_t head_off = (uint32_t)(g * D * 2);

  char* vbuf = smem + wave * attn_mfma_vbuf_bytes<D>();
  float m = -INFINITY, l = 0.f;  // head li
  attn_f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = attn_f32x4{0.f, 0.f, 0.f, 0.f};

  // Token of entry li of each tile (-1: none), polled when the indices come
  // from this kernel.
  int tok[TPW];
  auto entry_of = [&](int tt, int r) { return (tt * kItemWaves + wave) * 16 + r; };
  int n_have = n_ent;
  bool more_left = LIST;
  for (int r0 = 0;;) {
  if constexpr (LIST) {
    if (r0 >= n_have) {  // uniform
      if (!more_left) break;
      more_left = false;
      n_have = more();
      if (r0 >= n_have) break;
    }
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int e = r0 + entry_of(tt, li);
      tok[tt] = e < n_have ? list[e] : -1;
    }
  } else if (text) {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int e = entry_of(tt, li);
      tok[tt] = e < n_ent ? e0 + e : -1;
    }
  } else if (wait) {
    const uint32_t* ib = a.idx_enc + (int64_t)b * a.k + e0;
    for (uint32_t n = 0;; ++n) {
      bool missing = false;
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        const int e = entry_of(tt, li);
        const uint32_t w = e < n_ent ? load_flag(ib + e) : 0u;
        tok[tt] = e < n_ent ? (int)w - 1 : -1;
        missing |= e < n_ent && w == 0u;
      }
      if (!__syncthreads_or(missing)) break;
      if (n + 1 >= a.spin_limit) {
        if (tid == 0) report_giveup(a.status, kGiveUpIndices);
        break;
      }
      __builtin_amdgcn_s_sleep(24);
    }
  } else if (a.idx) {
    const int32_t* ib = a.idx + (int64_t)b * a.k + e0;
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int e = entry_of(tt, li);
      tok[tt] = e < n_ent ? ib[e] : -1;
    }
  } else {  // no index list: the visual rows 0..k-1 themselves (a packed cache)
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int e = entry_of(tt, li);
      tok[tt] = e < n_ent ? e0 + e : -1;
    }
  }
  const int lim = text ? a.Tmax : a.N;  // tokens outside [0, lim) are skipped
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
    if (tok[tt] < 0 || tok[tt] >= lim) tok[tt] = -1;

  // All loads in flight: K slices (A operand: entry li, dims 32 s + 8 lg)
  // and V rows (entry VEPL*i + lane / VCH, 16 bytes at chunk lane % VCH).
  u32x4 kr[TPW][KS], vr[TPW][VLD];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const uint32_t ko = tok[tt] >= 0 ? (uint32_t)(tok[tt] * ts * 2) + head_off + 16 * lg : kBufOob;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kr[tt][s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, ko + (ko == kBufOob ? 0 : 64 * s), 0, kCacheDefault));
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int vt = __shfl(tok[tt], VEPL * i + lane / VCH, kWave);
      const uint32_t vo = vt >= 0 ? (uint32_t)(vt * ts * 2) + head_off + 16 * (lane % VCH) : kBufOob;
      vr[tt][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, vo, 0, kCacheDefault));
    }
  }

#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    // Entries of this tile that count (bit r: entry r).
    const uint32_t valid = (uint32_t)__ballot(tok[tt] >= 0) & 0xFFFFu;
    if (!__builtin_amdgcn_readfirstlane(valid)) continue;  // uniform
#pragma unroll
    for (int i = 0; i < VLD; ++i)
      *reinterpret_cast<u32x4*>(vbuf + (VEPL * i + lane / VCH) * VSTR + 16 * (lane % VCH)) = vr[tt][i];
    attn_f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(attn_bf16x8, kr[tt][s]), qf[s], st, 0, 0, 0);
    // st[r] = S[head li][entry 4 lg + r]
    float x[4], tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = (valid >> (4 * lg + r)) & 1u ? st[r] * a.qscale : -INFINITY;
      tmax = fmaxf(tmax, x[r]);
    }
    tmax = fmaxf(tmax, xor_partner<16>(tmax));
    tmax = fmaxf(tmax, xor_partner<32>(tmax));
    const float mn = fmaxf(m, tmax);
    const float al = mn == -INFINITY ? 1.f : fast_exp2(m - mn);
    float pr[4], ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = x[r] == -INFINITY ? 0.f : fast_exp2(x[r] - mn);
      ps += pr[r];
    }
    l = l * al + ps;
    m = mn;
    if (__builtin_amdgcn_ballot_w64(al != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= al;
    }
    attn_s16x4 ph, pl;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint16_t h = attn_bf16_rne(pr[r]);
      ph[r] = (short)h;
      pl[r] = (short)attn_bf16_rne(pr[r] - __uint_as_float((uint32_t)h << 16));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      // V^T fragment: lane (li, lg) gets dim 16 db + li of entries 4 lg .. 4 lg + 3.
      const char* va = vbuf + (4 * lg + (li >> 2)) * VSTR + (16 * db + 4 * (li & 3)) * 2;
      const attn_s16x4 vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) attn_s16x4*)(va));
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, ph, acc[db], 0, 0, 0);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pl, acc[db], 0, 0, 0);
      // acc[db][r] = O[head li][dim 16 db + 4 lg + r]
    }
  }
  if constexpr (!LIST) break;
  r0 = r0 + SE < n_have ? r0 + SE : n_have;
  }
  l += xor_partner<16>(l);
  l += xor_partner<32>(l);

  // Slots of the vector front's cross-wave merge (the V buffers are done).
  __syncthreads();
  float* s_w = reinterpret_cast<float*>(smem);
  if (li < G) {
    float* sp = s_w + ((int64_t)wave * G + li) * (D + 2);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) sp[16 * db + 4 * lg + r] = acc[db][r];
    if (lg == 0) {
      sp[D] = m;
      sp[D + 1] = l;
    }
  }
}

struct NoMore {
  __device__ int operator()() const { return 0; }
};

// Item (b, g, c).  wait: the visual indices are produced by this kernel;
// poll their encoded copy idx_enc (bounded).  LIST: split c covers the visual
// tokens list[0 .. n_list) (LDS) and whatever more() appends after them (see
// attn_front_mfma), in rounds of the split's entry count.
template <typename T, int D, int G, int EPL, bool LIST = false, class More = NoMore>
__device__ __forceinline__ void attn_item(const AttnArgs& a, int b, int g, int c, bool wait,
                                          char* smem, const int* list = nullptr, int n_list = 0,
                                          More&& more = More{}) {
  using S = AttnShape<T, D>;
  constexpr int VE = S::VE, LPE = S::LPE, EPW = S::EPW;
  constexpr int SE = kItemWaves * EPW * EPL;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_uniform(tid / kWave);
  const int eg = lane / LPE, sub = lane % LPE, d0 = sub * VE;
  const T* q = reinterpret_cast<const T*>(a.q);
  const int C = a.CT + a.CV;

  const bool text = !LIST && c < a.CT;
  int n_ent;  // entries of this split
  int e0;     // first entry: text row or position in idx[b]
  if (LIST) {
    e0 = 0;
    n_ent = n_list;
  } else if (text) {
    int tl = a.txt_len ? a.txt_len[b] : 0;
    tl = tl < 0 ? 0 : (tl > a.Tmax ? a.Tmax : tl);
    e0 = c * SE;
    n_ent = tl - e0;
  } else {
    e0 = (c - a.CT) * SE;
    n_ent = a.k - e0;
  }
  n_ent = n_ent < 0 ? 0 : (!LIST && n_ent > SE ? SE : n_ent);

  float* s_w = reinterpret_cast<float*>(smem);
  auto slot = [&](int w, int i) { return s_w + ((int64_t)w * G + i) * (D + 2); };
  constexpr bool kMfma = std::is_same<T, bf16_t>::value && G >= 2;
  if constexpr (kMfma) {
    attn_front_mfma<D, G, SE, LIST>(a, b, g, text, e0, n_ent, wait, smem, list, more);
  } else {
    Vec<T> qx[G];
#pragma unroll
    for (int i = 0; i < G; ++i) qx[i].load(q + ((int64_t)b * a.Hq + g * G + i) * D + d0);

    // The sequence's text or visual cache as one buffer; entry j of this lane
    // is the head-g row of one token, at a 32-bit byte offset (kBufOob: none).
    constexpr int ES = (int)sizeof(T);
    const int64_t row_elems = (int64_t)a.Hkv * D;
    BufRsrc krs, vrs;
    int64_t ts;
    if (text) {
      ts = a.tts;
      const uint32_t ext = (uint32_t)(((int64_t)(a.Tmax > 0 ? a.Tmax - 1 : 0) * ts + row_elems) * ES);
      krs = make_rsrc(reinterpret_cast<const char*>(a.kt) + (int64_t)b * a.tbs * ES, ext);
      vrs = make_rsrc(reinterpret_cast<const char*>(a.vt) + (int64_t)b * a.tbs * ES, ext);
    } else {
      ts = a.vts;
      const uint32_t ext = (uint32_t)(((int64_t)(a.N > 0 ? a.N - 1 : 0) * ts + row_elems) * ES);
      krs = make_rsrc(reinterpret_cast<const char*>(a.kv) + (int64_t)b * a.vbs * ES, ext);
      vrs = make_rsrc(reinterpret_cast<const char*>(a.vv) + (int64_t)b * a.vbs * ES, ext);
    }
    const uint32_t head_off = (uint32_t)((g * D + d0) * ES);
    float qv[G][VE];
    float m[G], l[G], acc[G][VE];
    auto init = [&]() {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        qx[i].to_f32(qv[i]);
#pragma unroll
        for (int v = 0; v < VE; ++v) qv[i][v] *= a.qscale;
        m[i] = -INFINITY;
        l[i] = 0.f;
#pragma unroll
        for (int v = 0; v < VE; ++v) acc[i][v] = 0.f;
      }
    };
    if constexpr (LIST) init();
    int n_have = n_ent;
    bool more_left = LIST;
    for (int r0 = 0, it = 0;; ++it) {
    uint32_t off[EPL];
    if constexpr (LIST) {
      if (r0 >= n_have) {  // uniform
        if (!more_left) break;
        more_left = false;
        n_have = more();
        if (r0 >= n_have) break;
      }
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = r0 + (j * kItemWaves + wave) * EPW + eg;
        const int t = e < n_have ? list[e] : -1;
        off[j] = (t >= 0 && t < a.N) ? (uint32_t)(t * ts * ES) + head_off : kBufOob;
      }
    } else if (text) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = (j * kItemWaves + wave) * EPW + eg;
        off[j] = e < n_ent ? (uint32_t)((e0 + e) * ts * ES) + head_off : kBufOob;
      }
    } else {
      int tok[EPL];
      if (wait) {
        // The indices are produced by this kernel: poll this split's words of
        // the encoded copy until every one is written (bounded); the read that
        // finds them complete is the one that loads them.
        const uint32_t* ib = a.idx_enc + (int64_t)b * a.k + e0;
        for (uint32_t n = 0;; ++n) {
          bool missing = false;
#pragma unroll
          for (int j = 0; j < EPL; ++j) {
            const int e = (j * kItemWaves + wave) * EPW + eg;
            const uint32_t w = e < n_ent ? load_flag(ib + e) : 0u;
            tok[j] = e < n_ent ? (int)w - 1 : -1;  // -1: no entry
            missing |= e < n_ent && w == 0u;
          }
          if (!__syncthreads_or(missing)) break;
          if (n + 1 >= a.spin_limit) {
            if (tid == 0) report_giveup(a.status, kGiveUpIndices);
            break;
          }
          __builtin_amdgcn_s_sleep(24);
        }
      } else if (a.idx) {
        const int32_t* ib = a.idx + (int64_t)b * a.k + e0;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
          const int e = (j * kItemWaves + wave) * EPW + eg;
          tok[j] = e < n_ent ? ib[e] : -1;
        }
      } else {  // no index list: the visual rows 0..k-1 themselves (a packed cache)
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
          const int e = (j * kItemWaves + wave) * EPW + eg;
          tok[j] = e < n_ent ? e0 + e : -1;
        }
      }
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int t = tok[j];  // indices outside [0, N) are skipped
        off[j] = (t >= 0 && t < a.N) ? (uint32_t)(t * ts * ES) + head_off : kBufOob;
      }
    }

    Vec<T> kx[EPL], vx[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      kx[j].template load_buf<kCacheDefault>(krs, off[j], 0u);
      vx[j].template load_buf<kCacheDefault>(vrs, off[j], 0u);
    }

    if (!LIST && it == 0) init();  // after the loads are issued

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
        z[i] = lane_group_sum<LPE>(s);
      }
      // No entry (offset past the extent, zeros loaded): weight 0, state kept.
      // Selects, not a branch, so every load stays where it is issued.
      const bool valid = off[j] != kBufOob;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float mn = valid ? fmaxf(m[i], z[i]) : m[i];
        const float al = valid ? fast_exp2(m[i] - mn) : 1.f;  // m = -inf -> 0
        const float p = valid ? fast_exp2(z[i] - mn) : 0.f;
        l[i] = l[i] * al + p;
#pragma unroll
        for (int v = 0; v < VE; ++v) acc[i][v] = fmaf(p, vf[v], acc[i][v] * al);
        m[i] = mn;
      }
    }
    if constexpr (!LIST) break;
    r0 = r0 + SE < n_have ? r0 + SE : n_have;
    }

    // Merge the EPW lane groups of this wave (partner values by DPP and
    // row-swap moves, no LDS trips).
    auto merge_groups = [&](auto off_tag) {
      constexpr int OFF = decltype(off_tag)::value;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float mo = xor_partner<OFF>(m[i]);
        const float lo = xor_partner<OFF>(l[i]);
        const float mn = fmaxf(m[i], mo);
        const float al = (m[i] == -INFINITY) ? 0.f : fast_exp2(m[i] - mn);
        const float bo = (mo == -INFINITY) ? 0.f : fast_exp2(mo - mn);
        l[i] = l[i] * al + lo * bo;
#pragma unroll
        for (int v = 0; v < VE; ++v) {
          const float ao = xor_partner<OFF>(acc[i][v]);
          acc[i][v] = acc[i][v] * al + ao * bo;
        }
        m[i] = mn;
      }
    };
    if constexpr (LPE <= 8) merge_groups(std::integral_constant<int, 8>{});
    if constexpr (LPE <= 16) merge_groups(std::integral_constant<int, 16>{});
    if constexpr (LPE <= 32) merge_groups(std::integral_constant<int, 32>{});
    // Merge the waves through LDS: per wave and head, acc[D] then (m, l).
    if (eg == 0) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        float* sp = slot(wave, i);
#pragma unroll
        for (int v = 0; v < VE; ++v) sp[d0 + v] = acc[i][v];
        if (sub == 0) {
          sp[D] = m[i];
          sp[D + 1] = l[i];
        }
      }
    }
  }
  __syncthreads();
  const int64_t head0 = (int64_t)b * a.Hq + g * G;
  constexpr int PS = attn_part_stride(D);
  for (int t = tid; t < G * D; t += kItemThreads) {
    const int i = t / D, d = t % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kItemWaves; ++w) mm = fmaxf(mm, slot(w, i)[D]);
    float ll = 0.f, aa = 0.f;
#pragma unroll
    for (int w = 0; w < kItemWaves; ++w) {
      const float mw = slot(w, i)[D];
      const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - mm);
      ll += slot(w, i)[D + 1] * f;
      aa += slot(w, i)[d] * f;
    }
    if (C == 1) {
      a.out[(head0 + i) * D + d] = ll > 0.f ? aa / ll : 0.f;
    } else {
      float* pp = a.part + ((head0 + i) * C + c) * PS;
      store_shared_dev(pp + d, aa);
      if (d == 0) {
        store_shared_dev(pp + D, mm);
        store_shared_dev(pp + D + 1, ll);
      }
    }
  }
  if (C == 1) return;

  __shared__ uint32_t s_comb;
  wait_stores_complete();
  __syncthreads();
  uint32_t* ctr = a.comb_ctr + ((int64_t)b * a.Hkv + g) * kCtrStride;
  if (tid == 0) s_comb = counter_add(ctr, 1u) == (uint32_t)C - 1 ? 1u : 0u;
  __syncthreads();
  if (!s_comb) return;

  // out = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c, M = max_c m_c.
  const float* pb = a.part + head0 * C * PS;  // this (b, g): [G][C][PS]
  constexpr int V1 = G * D / 4;
  constexpr bool kOnline = LIST && kMfma && combine_groups<D, G>() == 1;
  constexpr int CB1 = 20;
  if (kOnline && C <= CB1) {
    // Chunk attention (few splits, one thread per float4 column): each thread
    // loads its column and (m, l) of every split in one round trip and merges
    // them online, rescaling as the maximum rises; no LDS and no barrier.
    if (tid < V1) {
      const int i = tid / (D / 4), d4 = tid % (D / 4);
      const BufRsrc pr = make_rsrc(pb, (uint32_t)(G * C * PS * 4));
      const uint32_t col = (uint32_t)(i * C * PS + 4 * d4) * 4u;
      const float* mlp = pb + (int64_t)i * C * PS + D;
      f32x4v x[CB1];
      float mc[CB1], lc[CB1];
#pragma unroll
      for (int j = 0; j < CB1; ++j) {
        x[j] = __builtin_bit_cast(f32x4v, load4_dev(pr, j < C ? col + (uint32_t)(j * PS * 4) : kBufOob));
        mc[j] = j < C ? load_shared_dev(mlp + (int64_t)j * PS) : -INFINITY;
        lc[j] = j < C ? load_shared_dev(mlp + (int64_t)j * PS + 1) : 0.f;
      }
      float M = -INFINITY, den = 0.f;
      f32x4v num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < CB1; ++j) {
        if (mc[j] != -INFINITY) {
          const float mn = fmaxf(M, mc[j]);
          const float a0 = M == -INFINITY ? 0.f : fast_exp2(M - mn);
          const float a1 = fast_exp2(mc[j] - mn);
          num = num * a0 + a1 * x[j];
          den = den * a0 + a1 * lc[j];
          M = mn;
        }
      }
      float* o = a.out + (head0 + i) * D + 4 * d4;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = den > 0.f ? num[j] / den : 0.f;
    }
  } else if (C <= 4 * combine_groups<D, G>()) {
    // Up to 4 splits per thread: thread (v, s) loads column v and (m, l) of
    // splits s, s + S, ... in one round trip and merges them online; the S
    // groups of a column then meet once in LDS.
    constexpr int S = combine_groups<D, G>();
    const int v = tid % V1, s = tid / V1;
    const int i = v / (D / 4), d4 = v % (D / 4);
    const BufRsrc pr = make_rsrc(pb, (uint32_t)(G * C * PS * 4));
    const uint32_t col = (uint32_t)(i * C * PS + 4 * d4) * 4u;
    const float* mlp = pb + (int64_t)i * C * PS + D;
    f32x4v x[4];
    float mc[4], lc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cc = s + j * S;
      const bool ok = s < S && cc < C;
      x[j] = __builtin_bit_cast(f32x4v, load4_dev(pr, ok ? col + (uint32_t)(cc * PS * 4) : kBufOob));
      mc[j] = ok ? load_shared_dev(mlp + (int64_t)cc * PS) : -INFINITY;
      lc[j] = ok ? load_shared_dev(mlp + (int64_t)cc * PS + 1) : 0.f;
    }
    float M = -INFINITY, den = 0.f;
    f32x4v num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (mc[j] != -INFINITY) {
        const float mn = fmaxf(M, mc[j]);
        const float a0 = M == -INFINITY ? 0.f : fast_exp2(M - mn);
        const float a1 = fast_exp2(mc[j] - mn);
        num = num * a0 + a1 * x[j];
        den = den * a0 + a1 * lc[j];
        M = mn;
      }
    }
    if constexpr (S > 1) {
      f32x4v* s_num = reinterpret_cast<f32x4v*>(smem);  // [S][V]
      float* s_m = reinterpret_cast<float*>(s_num + S * V1);
      float* s_d = s_m + S * V1;
      if (s < S) {
        s_num[tid] = num;
        s_m[tid] = M;
        s_d[tid] = den;
      }
      __syncthreads();
      if (s == 0) {
        float Mt = M;
#pragma unroll
        for (int r = 1; r < S; ++r) Mt = fmaxf(Mt, s_m[r * V1 + v]);
        const float f0 = M == -INFINITY ? 0.f : fast_exp2(M - Mt);
        num = num * f0;
        den = den * f0;
#pragma unroll
        for (int r = 1; r < S; ++r) {
          const float mr = s_m[r * V1 + v];
          const float fr = mr == -INFINITY ? 0.f : fast_exp2(mr - Mt);
          num += fr * s_num[r * V1 + v];
          den += fr * s_d[r * V1 + v];
        }
      }
    }
    if (s == 0) {
      float* o = a.out + (head0 + i) * D + 4 * d4;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = den > 0.f ? num[j] / den : 0.f;
    }
  } else if (C <= kMaxCombineSplits) {
    // Thread (v, s) sums float4 column v over splits s, s+S, ...; its first
    // 8 loads go out together with the (m, l) loads of every split (to LDS),
    // so up to 8 S splits merge in one round trip (8, not more: the batch's
    // registers set the fused kernel's occupancy).  Then one wave per head turns
    // m into the weight 2^(m - M) and sums the denominator, and the S groups
    // of a column meet in LDS.
    float* s_f = reinterpret_cast<float*>(smem);  // [G][C]
    float* s_l = s_f + G * kMaxCombineSplits;    // [G][C]
    float* s_den = s_l + G * kMaxCombineSplits;  // [G]
    f32x4v* s_red = reinterpret_cast<f32x4v*>(s_den + 8);
    constexpr int V = G * D / 4, S = combine_groups<D, G>();
    const int v = tid % V, s = tid / V;
    const int i = v / (D / 4), d4 = v % (D / 4);
    const BufRsrc pr = make_rsrc(pb, (uint32_t)(G * C * PS * 4));
    const uint32_t col = (uint32_t)(i * C * PS + 4 * d4) * 4u;
    auto col_load = [&](int cc) {
      return __builtin_bit_cast(
          f32x4v, load4_dev(pr, (s < S && cc < C) ? col + (uint32_t)(cc * PS * 4) : kBufOob));
    };
    f32x4v x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = col_load(s + j * S);
    for (int t = tid; t < G * C; t += kItemThreads) {
      s_f[t] = load_shared_dev(pb + (int64_t)t * PS + D);
      s_l[t] = load_shared_dev(pb + (int64_t)t * PS + D + 1);
    }
    __syncthreads();
    for (int h = wave; h < G; h += kItemWaves) {
      float M = -INFINITY;
      for (int cc = lane; cc < C; cc += kWave) M = fmaxf(M, s_f[h * C + cc]);
      M = group_max<kWave>(M);
      float den = 0.f;
      for (int cc = lane; cc < C; cc += kWave) {
        const float mc = s_f[h * C + cc];
        const float f = (mc == -INFINITY) ? 0.f : fast_exp2(mc - M);
        s_f[h * C + cc] = f;
        den = fmaf(f, s_l[h * C + cc], den);
      }
      den = group_sum<kWave>(den);
      if (lane == 0) s_den[h] = den;
    }
    __syncthreads();
    f32x4v num = {0.f, 0.f, 0.f, 0.f};
    const float* fw = s_f + i * C;
    for (int c0 = s;; c0 += 8 * S) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int cc = c0 + j * S;
        num += (s < S && cc < C ? fw[cc] : 0.f) * x[j];
      }
      if (c0 + 8 * S >= C) break;  // no barrier inside: per-thread exit is fine
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = col_load(c0 + 8 * S + j * S);
    }
    if constexpr (S > 1) {
      s_red[tid] = num;
      __syncthreads();
      if (s == 0) {
#pragma unroll
        for (int r = 1; r < S; ++r) num += s_red[r * V + v];
      }
    }
    if (s == 0 && tid < V) {
      const float den = s_den[i];
      float* o = a.out + (head0 + i) * D + 4 * d4;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = den > 0.f ? num[j] / den : 0.f;
    }
  } else {
    // More splits than LDS holds: read (m, l) in place.
    for (int t = tid; t < G * D; t += kItemThreads) {
      const int i = t / D, d = t % D;
      const float* pp = pb + (int64_t)i * C * PS;
      float M = -INFINITY;
      for (int cc = 0; cc < C; ++cc) M = fmaxf(M, load_shared_dev(pp + cc * PS + D));
      float num = 0.f, den = 0.f;
      if (M != -INFINITY) {
#pragma unroll 8
        for (int cc = 0; cc < C; ++cc) {
          const float mc = load_shared_dev(pp + cc * PS + D);
          const float f = (mc == -INFINITY) ? 0.f : fast_exp2(mc - M);
          num = fmaf(f, load_shared_dev(pp + cc * PS + d), num);
          den = fmaf(f, load_shared_dev(pp + cc * PS + D + 1), den);
        }
      }
      a.out[(head0 + i) * D + d] = den > 0.f ? num / den : 0.f;
    }
  }
  if (tid == 0) counter_reset(ctr);
}

// Entries per split for (dtype, D, EPL).
__host__ inline int attn_split_entries(int VE, int D, int EPL) {
  return kItemWaves * (kWave / (D / VE)) * EPL;
}

}  // namespace sv
