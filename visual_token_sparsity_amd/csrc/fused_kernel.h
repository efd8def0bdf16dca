// One decode layer in one launch: relevance scan, exact top-k, sparse
// attention over the selected visual entries plus the text entries, and the
// split combine (SparseVILA velog summary, Sec. 3.2 and Sec. 4.5).
//
// Work order.  Workgroup i runs item i, in this order:
//   rows that fit the select's registers: for each sequence b, its scan
//     items, then its select item;
//   longer rows (the parallel select of long_select.h, P = ceil(N / 2048)
//     chunks per row): every scan item of every sequence, then the P
//     candidate items of each sequence, the threshold items, and the P
//     compaction items of each sequence;
//   the text attention items (they need no selection);
//   the visual attention items, sequence by sequence (each polls the words
//     of the encoded index copy it needs).
// Short rows: there are more scan items than resident workgroups, so the
// sequences finish their scans one after another and each select overlaps
// the scans of the sequences behind it.  Scan items store each score
// complemented (a zero word: not written yet) and never wait; the select
// item of b polls the score row until it is complete, which also loads its
// keys.  Long rows: the select items come after all scan items, so none of
// them holds a workgroup slot while scans still wait for one.
//
// Each XCD dispatches its share of the grid in increasing order, so whatever
// a waiting workgroup waits on has been dispatched before it, and scan items
// never wait.  All waits are bounded.  No atomic ticket: same-address
// atomics from thousands of workgroups serialise in the memory system.
//
// Control words (one 128-byte line each) are zero after every launch:
// the scan count lines of b by the selecting workgroup (long rows: the
// threshold item), comb_ctr[b,g] by the combining one, and vis_done[b] counts visual
// items past their wait, the last of which lowers ready[b] again and clears
// the encoded index copy the visual items poll.
// Complemented scores are zeroed by the select item that read them; the
// long-row histograms and counters by the threshold and compaction items.
#pragma once

#include "long_select.h"

namespace sv {

struct FusedCtl {
  uint32_t B;
  uint32_t per_seq;    // short rows: scan items + 1 select item per sequence
  uint32_t seq_end;    // items before the attention items
  uint32_t text_end, total;
  bool auto_rows;      // long rows: size the scan items from the kernel's occupancy
  uint32_t* vis_done;
  float* scores_out;   // decoded scores (polling mode), may be null
};

// LDS of a chunk attention item: the attention item's, then the chunk's token
// list and kItemWaves + 2 words.
template <int D, int G>
__host__ __device__ constexpr size_t chunk_list_offset() {
  return (attn_smem_bytes<D, G>() + 15) & ~(size_t)15;
}
template <int D, int G>
__host__ __device__ constexpr size_t chunk_attn_smem_bytes() {
  return chunk_list_offset<D, G>() + (size_t)kLsChunk * 4 + (kItemWaves + 2) * 4;
}

// Long rows, chunk attention: the item of (b, g, p) attends over the selected
// tokens of score chunk p, the keys above D1 first (as soon as D1 is
// published), then those of digit D1 under the threshold (once it is).  The
// compaction items still write idx[b] but no longer gate the attention.
template <typename T, int D, int G, int EPL>
__device__ __forceinline__ void chunk_attn_item(const ScanArgs& sa, const AttnArgs& aa,
                                                const LongSelArgs& ls, int b, int g, int p,
                                                char* smem) {
  int* list = reinterpret_cast<int*>(smem + chunk_list_offset<D, G>());
  uint32_t* wcnt = reinterpret_cast<uint32_t*>(list + kLsChunk);
  const int tid = threadIdx.x;
  ChunkSel cs;
  if (tid == 0)
    wcnt[kItemWaves] = poll_until(ls_line(ls, b, kLsInfo1) + 3, 1u, sa.spin_limit, sa.status,
                                  kGiveUpIndices) - 1u;
  __syncthreads();
  cs.D1 = wcnt[kItemWaves];
  load_chunk_keys(sa.scores, sa.N, b, p, cs.key, cs.e0);
  cs.cend = min(sa.N, (p + 1) * kLsChunk);
  const int n1 = chunk_list_append(cs, list, wcnt, 0, false, 0u, 0u);
  auto more = [&]() -> int {
    if (tid == 0) {
      // The threshold element, published as one word T | (Ti + 1) << 32.
      const uint64_t* pub = thr_pub_word(ls, b);
      uint64_t w = 0;
      for (uint32_t n = 0; n < sa.spin_limit; ++n) {
        w = __hip_atomic_load(pub, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (w) break;
        __builtin_amdgcn_s_sleep(2);
      }
      if (!w) report_giveup(sa.status, kGiveUpThreshold);
      wcnt[kItemWaves] = (uint32_t)w;
      wcnt[kItemWaves + 1] = (uint32_t)(w >> 32) - 1u;
      threshold_read_done(ls, b);
    }
    __syncthreads();
    const uint32_t tkey = wcnt[kItemWaves], tidx = wcnt[kItemWaves + 1];
    return chunk_list_append(cs, list, wcnt, n1, true, tkey, tidx);
  };
  attn_item<T, D, G, EPL, true>(aa, b, g, aa.CT + p, false, smem, list, n1, more);
}

// LONG: rows of more than 2048 tokens (the parallel select); each mode is
// its own instantiation, so neither carries the other's registers.
template <typename T, int D, int G, int EPL, bool LONG>
__global__ __launch_bounds__(kItemThreads) void fused_kernel(ScanArgs sa, AttnArgs aa,
                                                             FusedCtl ctl, LongSelArgs ls) {
  extern __shared__ __align__(16) char smem[];
  const uint32_t t = blockIdx.x;
  if (t < ctl.seq_end) {
    int q_of = -1;
    if constexpr (!LONG) {
      const int b = wave_uniform(t / ctl.per_seq);
      const int j = wave_uniform(t % ctl.per_seq);
      if (j < sa.items_per_seq) {
        // Scores stored complemented (encode): the scan item never selects,
        // the select item below does.
        scan_item<T, short_scan_cpl<T>()>(sa, b, j, smem, q_of);
      } else {
        select_poll_item(sa, b, ctl.scores_out, smem);
      }
      return;
    }
    const uint32_t S = (uint32_t)sa.items_per_seq, P = (uint32_t)ls.P;
    uint32_t u = t;
    if (u < ctl.B * S) {
      // G >= 2: the attention items set the registers, so the scan can pair rows.
      scan_item<T, kScanCpl, (G >= 2)>(sa, wave_uniform(u / S), wave_uniform(u % S), smem, q_of);
    } else if ((u -= ctl.B * S) < ctl.B * P) {
      cand_item(sa, ls, wave_uniform(u / P), wave_uniform(u % P), smem);
    } else if ((u -= ctl.B * P) < ctl.B) {
      thr_item(sa, ls, u, smem);
    } else {
      u -= ctl.B;
      compact_item(sa, ls, wave_uniform(u / P), wave_uniform(u % P), smem);
    }
    return;
  }
  const bool text = t < ctl.text_end;
  uint32_t u = text ? t - ctl.seq_end : t - ctl.text_end;
  if constexpr (LONG) {
    if (!text && ls.chunk_attn) {
      const uint32_t P = (uint32_t)ls.P;
      chunk_attn_item<T, D, G, EPL>(sa, aa, ls, wave_uniform(u / (P * aa.Hkv)),
                                    wave_uniform((u / P) % aa.Hkv), wave_uniform(u % P), smem);
      return;
    }
  }
  const int per = text ? aa.CT : aa.CV;
  const int b = wave_uniform(u / (per * aa.Hkv));
  const int g = wave_uniform((u / per) % aa.Hkv);
  attn_item<T, D, G, EPL>(aa, b, g, wave_uniform((text ? 0 : aa.CT) + u % per), !text, smem);
  if (text) return;
  // The last visual item of b (every other one has read its indices) clears
  // the encoded index copy, ready[b] and the count for the next launch.
  __shared__ uint32_t s_last;
  uint32_t* vd = ctl.vis_done + b * kCtrStride;
  if (threadIdx.x == 0) s_last = counter_add(vd, 1u) == (uint32_t)(aa.CV * aa.Hkv) - 1 ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  uint32_t* enc = const_cast<uint32_t*>(aa.idx_enc) + (int64_t)b * aa.k;
  for (int i = threadIdx.x; i < aa.k; i += kItemThreads) store_flag(enc + i, 0u);
  if (threadIdx.x == 0) {
    store_flag(aa.ready + b * kCtrStride, 0u);
    counter_reset(vd);
  }
}

template <typename T, int D, int G, int EPL, bool LONG>
static hipError_t fused_go(const ScanArgs& sa, const AttnArgs& aa, const FusedCtl& ctl,
                           const LongSelArgs& ls, hipStream_t st) {
  const int VE = Vec<T>::kElems;
  size_t lds = scan_smem_bytes(sa.nseg, sa.LPR, VE, LONG, LONG ? kScanCpl : short_scan_cpl<T>());
  if (attn_smem_bytes<D, G>() > lds) lds = attn_smem_bytes<D, G>();
  if (sa.hist1) {
    if (cand_smem_bytes() > lds) lds = cand_smem_bytes();
    if (thr_smem_bytes(ls.P) > lds) lds = thr_smem_bytes(ls.P);
    if (ls.chunk_attn && chunk_attn_smem_bytes<D, G>() > lds) lds = chunk_attn_smem_bytes<D, G>();
  }
  if (lds > 48 * 1024) {
    static bool raised = false;  // per instantiation; the attribute is per function
    if (!raised) {
      const hipError_t e = hipFuncSetAttribute((const void*)fused_kernel<T, D, G, EPL, LONG>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               96 * 1024);
      if (e != hipSuccess) return e;
      raised = true;
    }
  }
  if (lds > 96 * 1024) return hipErrorInvalidValue;
  ScanArgs s = sa;
  FusedCtl c = ctl;
  if (ctl.auto_rows) {
    // Long rows: one round of scan items, as many as fit on the device at
    // once (a second, partly filled round would leave the memory system
    // idle at its end).
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_kernel<T, D, G, EPL, LONG>,
                                                     kItemThreads, lds) == hipSuccess &&
        per_cu > 0) {
      const uint32_t attn_items = ctl.total - ctl.seq_end, text_items = ctl.text_end - ctl.seq_end;
      const uint32_t sel_items = ctl.per_seq - (uint32_t)sa.items_per_seq;
      s.rows_per_item = scan_rows_for_items((int)ctl.B, sa.N, sa.LPR, sa.nseg,
                                            (long)per_cu * device_cu_count());
      s.items_per_seq = (sa.N + s.rows_per_item - 1) / s.rows_per_item;
      c.per_seq = (uint32_t)s.items_per_seq + sel_items;
      c.seq_end = c.per_seq * ctl.B;
      c.text_end = c.seq_end + text_items;
      c.total = c.seq_end + attn_items;
    }
  }
  hipLaunchKernelGGL((fused_kernel<T, D, G, EPL, LONG>), dim3(c.total), dim3(kItemThreads), lds, st,
                     s, aa, c, ls);
  return hipGetLastError();
}

template <typename T, int D, int G, bool LONG>
static hipError_t fused_epl(int epl, const ScanArgs& sa, const AttnArgs& aa, const FusedCtl& ctl,
                            const LongSelArgs& ls, hipStream_t st) {
  switch (epl) {  // the fused launch plans 4 or 8 entries per lane
    case 4: return fused_go<T, D, G, 4, LONG>(sa, aa, ctl, ls, st);
    case 8: return fused_go<T, D, G, 8, LONG>(sa, aa, ctl, ls, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D, bool LONG>
static hipError_t fused_g(int G, int epl, const ScanArgs& sa, const AttnArgs& aa,
                          const FusedCtl& ctl, const LongSelArgs& ls, hipStream_t st) {
  switch (G) {
    case 1: return fused_epl<T, D, 1, LONG>(epl, sa, aa, ctl, ls, st);
    case 2: return fused_epl<T, D, 2, LONG>(epl, sa, aa, ctl, ls, st);
    case 3: return fused_epl<T, D, 3, LONG>(epl, sa, aa, ctl, ls, st);
    case 4: return fused_epl<T, D, 4, LONG>(epl, sa, aa, ctl, ls, st);
    case 5: return fused_epl<T, D, 5, LONG>(epl, sa, aa, ctl, ls, st);
    case 6: return fused_epl<T, D, 6, LONG>(epl, sa, aa, ctl, ls, st);
    case 7: return fused_epl<T, D, 7, LONG>(epl, sa, aa, ctl, ls, st);
    case 8: return fused_epl<T, D, 8, LONG>(epl, sa, aa, ctl, ls, st);
    default: return hipErrorInvalidValue;
  }
}

// One (dtype, row mode)'s instantiations, each compiled in a translation unit
// of its own so that they build in parallel.
template <typename T, bool LONG>
hipError_t launch_fused_typed(int D, int G, int epl, const ScanArgs& sa, const AttnArgs& aa,
                              const FusedCtl& ctl, const LongSelArgs& ls, hipStream_t st) {
  return D == 128 ? fused_g<T, 128, LONG>(G, epl, sa, aa, ctl, ls, st)
                  : fused_g<T, 64, LONG>(G, epl, sa, aa, ctl, ls, st);
}

}  // namespace sv
