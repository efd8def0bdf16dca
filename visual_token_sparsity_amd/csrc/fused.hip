// One decode layer in one launch: relevance scan, exact top-k, sparse
// attention over the selected visual entries plus the text entries, and the
// split combine (SparseVILA velog summary, Sec. 3.2 and Sec. 4.5).
//
// Work order.  Workgroup i runs item i, in this order:
//   for each sequence b: its scan items, then (rows that fit the select's
//     registers) its select item;
//   the text attention items (they need no selection);
//   the visual attention items, sequence by sequence (each polls ready[b]).
// There are more scan items than resident workgroups, so the sequences
// finish their scans one after another and each select overlaps the scans
// of the sequences behind it.  Scan items store each score complemented (a
// zero word: not written yet) and never wait; the select item of b polls
// the score row until it is complete, which also loads its keys.  Longer
// rows use counters instead: every scan item of b bumps seq_ctr[b] after
// its stores have completed, and the last one selects.
//
// Each XCD dispatches its share of the grid in increasing order, so whatever
// a waiting workgroup waits on has been dispatched before it, and scan items
// never wait.  All waits are bounded.  No atomic ticket: same-address
// atomics from thousands of workgroups serialise in the memory system.
//
// Control words (one 128-byte line each) are zero after every launch:
// seq_ctr[b] is reset by the selecting workgroup, comb_ctr[b,g] by the
// combining one, and vis_done[b] counts visual items past their wait, the
// last of which lowers ready[b] again.  Complemented scores are zeroed by
// the select item that read them.
#include "fused_kernel.h"

namespace sv {

// Defined in fused_bf16.hip and fused_f32.hip.
extern template hipError_t launch_fused_typed<bf16_t>(int, int, int, const ScanArgs&,
                                                      const AttnArgs&, const FusedCtl&, hipStream_t);
extern template hipError_t launch_fused_typed<float>(int, int, int, const ScanArgs&,
                                                     const AttnArgs&, const FusedCtl&, hipStream_t);

hipError_t launch_fused(const FusedLaunch& f, hipStream_t st) {
  const int VE = f.dtype == 1 ? 8 : 4;
  const int G = f.Hq / f.Hkv;
  ScanArgs sa{};
  sa.q = f.q;
  sa.Tq = 1;
  sa.Hq = f.Hq;
  sa.G = G;
  sa.kv = f.k_vis;
  sa.bstride = f.vbs;
  sa.tstride = f.vts;
  sa.N = f.N;
  sa.D = f.D;
  sa.C = f.Hkv * f.D / VE;
  scan_geometry(sa.C, &sa.nseg, &sa.LPR);
  // Rows that fit the select's registers: small scan items (more of them
  // than resident workgroups, so the sequences finish one after another),
  // complemented scores and a polling select item per sequence.
  sa.encode = f.N <= kItemThreads * kSelKpt;
  const int min_rows = kItemWaves * (sa.nseg > 1 ? 1 : kWave / sa.LPR);
  sa.rows_per_item = f.rows_per_item > 0 ? f.rows_per_item
                     : sa.encode       ? 2 * min_rows
                                       : scan_rows_per_item(f.B, f.N, sa.LPR, sa.nseg);
  sa.items_per_seq = (f.N + sa.rows_per_item - 1) / sa.rows_per_item;
  sa.scores = sa.encode ? f.scores_ws : (f.scores_out ? f.scores_out : f.scores_ws);
  sa.k = f.k;
  sa.idx = f.idx;
  sa.seq_ctr = f.seq_ctr;
  sa.ready = f.ready;

  AttnPlan p = fused_attn_plan(f.B, f.Hkv, f.D, VE, f.k, f.Tmax);
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

  FusedCtl ctl{};
  ctl.vis_done = f.vis_done;
  ctl.scores_out = sa.encode ? f.scores_out : nullptr;
  ctl.per_seq = (uint32_t)sa.items_per_seq + (sa.encode ? 1u : 0u);
  ctl.seq_end = ctl.per_seq * (uint32_t)f.B;
  ctl.text_end = ctl.seq_end + (uint32_t)p.CT * f.Hkv * f.B;
  ctl.total = ctl.text_end + (uint32_t)p.CV * f.Hkv * f.B;
  if (f.dtype == 1) return launch_fused_typed<bf16_t>(f.D, G, p.EPL, sa, aa, ctl, st);
  return launch_fused_typed<float>(f.D, G, p.EPL, sa, aa, ctl, st);
}

}  // namespace sv
