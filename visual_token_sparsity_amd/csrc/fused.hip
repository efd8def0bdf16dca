// Host side of the one-launch decode layer: the work plan of one launch and
// the long-row select workspace (the kernel and its work order are in
// fused_kernel.h; SparseVILA velog summary, Sec. 3.2 and Sec. 4.5).
#include "fused_kernel.h"

namespace sv {

// Defined in fused_bf16.hip, fused_bf16_long.hip, fused_f32.hip and fused_f32_long.hip.
#define SV_FUSED_EXTERN(T, LONG)                                                          \
  extern template hipError_t launch_fused_typed<T, LONG>(int, int, int, const ScanArgs&,   \
                                                        const AttnArgs&, const FusedCtl&, \
                                                        const LongSelArgs&, hipStream_t)
SV_FUSED_EXTERN(bf16_t, false);
SV_FUSED_EXTERN(bf16_t, true);
SV_FUSED_EXTERN(float, false);
SV_FUSED_EXTERN(float, true);
#undef SV_FUSED_EXTERN

// Long-row select workspace, per launch:
//   [ctl B*kLsCtlLines lines][scan counts B*kLsScanCtrs lines][hist1 B*kLsReps*kLsBins]
//   [hist2 B*kLsBins]  (zero between launches)
//   [cand B*kLsCandCap][chunk_hi B*P][offs B*P]
static size_t al256(size_t n) { return (n + 255) & ~(size_t)255; }
static bool long_rows(int N) { return N > kItemThreads * kSelKpt; }
static int long_chunks(int N) { return (N + kLsChunk - 1) / kLsChunk; }

// Chunk attention items, B*Hkv*P of them, each reading its 2048 scores: worth
// it where they are few (a batch-1 video layer: 52), not for 128k-token rows
// of many heads (8192 of them, one 8 KB score read each).
constexpr long kChunkAttnMaxItems = 1024;
static_assert(kLsChunk == 2048, "fused_attn_plan counts chunks of 2048 scores");

bool fused_chunk_attn(int B, int Hkv, int N, int k) {
  return long_rows(N) && k > 0 && (long)B * Hkv * long_chunks(N) <= kChunkAttnMaxItems;
}

size_t long_select_zero_bytes(int B, int N) {
  if (!long_rows(N)) return 0;
  return al256((size_t)B * kLsCtlLines * kCtrStride * 4) +
         al256((size_t)B * kLsScanCtrs * kCtrStride * 4) +
         al256((size_t)B * kLsReps * kLsBins * 4) + al256((size_t)B * kLsBins * 4);
}

size_t long_select_bytes(int B, int N) {
  if (!long_rows(N)) return 0;
  const size_t P = (size_t)long_chunks(N);
  return long_select_zero_bytes(B, N) + al256((size_t)B * kLsCandCap * 8) +
         2 * al256((size_t)B * P * 4);
}

hipError_t launch_fused(const FusedLaunch& f, hipStream_t st) {
  const int VE = f.dtype == 1 ? 8 : 4;
  const int G = f.Hq / f.Hkv;
  if (f.retrieve_only && !long_rows(f.N)) return hipErrorInvalidValue;
  ScanArgs sa{};
  sa.q = f.q;
  sa.Tq = f.Tq > 0 ? f.Tq : 1;
  sa.Hq = f.Hq;
  sa.G = G;
  sa.kv = f.k_vis;
  sa.bstride = f.vbs;
  sa.tstride = f.vts;
  sa.N = f.N;
  sa.D = f.D;
  sa.C = f.Hkv * f.D / VE;
  scan_geometry(sa.C, &sa.nseg, &sa.LPR, long_rows(f.N) ? kScanCpl : short_scan_cpl(f.dtype));
  // Rows that fit the select's registers: small scan items (more of them
  // than resident workgroups, so the sequences finish one after another),
  // complemented scores and a polling select item per sequence.  Longer
  // rows: the parallel select of long_select.h.
  sa.encode = !long_rows(f.N);
  const int min_rows = kItemWaves * (sa.nseg > 1 ? 1 : kWave / sa.LPR);
  sa.rows_per_item = f.rows_per_item > 0 ? f.rows_per_item
                     : sa.encode       ? 2 * min_rows
                                       : scan_rows_per_item(f.B, f.N, sa.LPR, sa.nseg);
  sa.items_per_seq = (f.N + sa.rows_per_item - 1) / sa.rows_per_item;
  sa.scores = sa.encode ? f.scores_ws : (f.scores_out ? f.scores_out : f.scores_ws);
  sa.k = f.k;
  sa.idx = f.idx;
  sa.seq_ctr = f.seq_ctr;
  sa.ready = f.retrieve_only ? nullptr : f.ready;
  sa.idx_enc = f.retrieve_only ? nullptr : f.idx_enc;
  sa.spin_limit = f.spin_limit > 0 ? f.spin_limit : kSpinLimit;
  sa.status = f.status;
  LongSelArgs ls{};
  if (!sa.encode) {
    if (!f.long_ws) return hipErrorInvalidValue;
    const size_t P = (size_t)long_chunks(f.N);
    char* w = static_cast<char*>(f.long_ws);
    ls.P = (int)P;
    ls.ctl = reinterpret_cast<uint32_t*>(w);
    w += al256((size_t)f.B * kLsCtlLines * kCtrStride * 4);
    sa.seq_ctr = reinterpret_cast<uint32_t*>(w);  // the scan items' count lines
    sa.ctr_log2 = kLsScanCtrLog2;
    w += al256((size_t)f.B * kLsScanCtrs * kCtrStride * 4);
    ls.hist1 = reinterpret_cast<uint32_t*>(w);
    w += al256((size_t)f.B * kLsReps * kLsBins * 4);
    ls.hist2 = reinterpret_cast<uint32_t*>(w);
    w += al256((size_t)f.B * kLsBins * 4);
    ls.cand = reinterpret_cast<uint64_t*>(w);
    w += al256((size_t)f.B * kLsCandCap * 8);
    ls.chunk_hi = reinterpret_cast<uint32_t*>(w);
    w += al256((size_t)f.B * P * 4);
    ls.offs = reinterpret_cast<uint32_t*>(w);
    sa.hist1 = ls.hist1;
    ls.chunk_attn = !f.retrieve_only && fused_chunk_attn(f.B, f.Hkv, f.N, f.k);
    ls.readers = (uint32_t)P * (ls.chunk_attn ? 1u + (uint32_t)f.Hkv : 1u);
    if (ls.chunk_attn) {
      // Neither the encoded index copy nor ready[b] is waited on.
      sa.idx_enc = nullptr;
      sa.ready = nullptr;
    }
  }

  AttnPlan p = fused_attn_plan(f.B, f.Hkv, f.D, VE, f.k, f.Tmax, f.N);
  if (f.epl > 0) {
    p.EPL = f.epl;
    p.SE = attn_split_entries(VE, f.D, f.epl);
    p.CT = (f.Tmax + p.SE - 1) / p.SE;
    p.CV = (f.k + p.SE - 1) / p.SE;
  }
  AttnArgs aa{};
  aa.q = f.q;
  aa.Hq = f.Hq;
  aa.Hkv = f.Hkv;
  aa.kv = f.k_vis;
  aa.vv = f.v_vis;
  aa.vbs = f.vbs;
  aa.vts = f.vts;
  aa.N = f.N;
  aa.idx = f.idx;
  aa.k = f.k;
  aa.kt = f.k_txt;
  aa.vt = f.v_txt;
  aa.tbs = f.tbs;
  aa.tts = f.tts;
  aa.txt_len = f.txt_len;
  aa.Tmax = f.Tmax;
  aa.qscale = f.scale * 1.4426950408889634f;
  aa.CT = p.CT;
  aa.CV = p.CV;
  aa.part = f.part;
  aa.comb_ctr = f.comb_ctr;
  aa.out = f.out;
  aa.ready = f.ready;
  aa.idx_enc = f.idx_enc;
  aa.spin_limit = sa.spin_limit;
  aa.status = f.status;

  FusedCtl ctl{};
  ctl.vis_done = f.vis_done;
  ctl.scores_out = sa.encode ? f.scores_out : nullptr;
  ctl.B = (uint32_t)f.B;
  ctl.auto_rows = !sa.encode && f.rows_per_item <= 0;
  ctl.per_seq = (uint32_t)sa.items_per_seq + (sa.encode ? 1u : 2u * (uint32_t)ls.P + 1u);
  ctl.seq_end = ctl.per_seq * (uint32_t)f.B;  // long rows: the same count, in phase order
  ctl.text_end = ctl.seq_end + (uint32_t)p.CT * f.Hkv * f.B;
  ctl.total = ctl.text_end + (uint32_t)p.CV * f.Hkv * f.B;
  if (f.retrieve_only) ctl.text_end = ctl.total = ctl.seq_end;
  const bool lng = sa.hist1 != nullptr;
  if (f.dtype == 1)
    return lng ? launch_fused_typed<bf16_t, true>(f.D, G, p.EPL, sa, aa, ctl, ls, st)
               : launch_fused_typed<bf16_t, false>(f.D, G, p.EPL, sa, aa, ctl, ls, st);
  return lng ? launch_fused_typed<float, true>(f.D, G, p.EPL, sa, aa, ctl, ls, st)
             : launch_fused_typed<float, false>(f.D, G, p.EPL, sa, aa, ctl, ls, st);
}

}  // namespace sv
