// Prefill attention of a question chunk with the query-aware retrieval fused
// into it.
//
// SparseVILA velog summary, Sec. 3.2 (query-aware token selection, its
// implementation note): the retrieval salience of the question is computed
// alongside the question's ordinary (FlashAttention) prefill attention; the
// kernel table (Sec. 3.3) credits the retrieval-salience kernel with its
// speedup.  Both need the same logits q . K of every question token against
// every visual key: the attention turns them into a causal softmax over the
// whole context, the retrieval sums them (raw) over the question's tokens and
// the query heads of each KV head.  Here one pass over the caches does both.
//
// Item (b, g, rc, c): KV head g of sequence b, row chunk rc of the question's
// Tq * G query rows of that head (row = tau * G + h % G), key split c (visual
// splits first, then text splits; E keys each).  W waves per workgroup, 32
// query rows per wave (two 16-row blocks).  Keys stream through LDS in
// stages of 32 (double-buffered): K fragment-major (direct global -> LDS
// loads), V row-major with a padded row stride.
//
//   S^T = K Q^T   (v_mfma_f32_16x16x32_bf16: A = K tile, B = Q^T, fp32 acc;
//                  lane (li, lg) holds keys 4 lg + r of row li)
//   retrieval:    raw S^T summed over the wave's rows (DPP over the 16 lanes
//                 of a key group) -> partial score of each visual key
//   softmax:      online, per row; x = S scale log2(e), masked (keys past the
//                 split, text rows past the token's position) to -inf
//   O^T += V^T P^T (v_mfma_f32_16x16x16_bf16: B = P^T straight from the S^T
//                  registers, as bf16 high part + bf16 residual; A = V^T read
//                  with ds_read_tr16_b64, which transposes 4 x 16-bit per lane)
//
// Partials (m, l, O) of each split go to the workspace; a combine kernel
// merges them per row by max-rescaling, and a third kernel sums the partial
// retrieval scores in a fixed order (deterministic) before the top-k select.
//
// Up to 32 query rows per KV head (one row block: a short question, or few
// query heads per KV head): eight waves share the item's row block and split
// its keys (wave w takes stages w, w + 8, ...), so an item has eight waves'
// worth of loads in flight and one partial.  K fragments go from memory
// straight into registers; V rows go through a private LDS buffer per wave.  The splits run over the sequence's keys as one list
// (visual, then text).  At the end the waves' (m, l, O) meet in LDS in a
// fixed order (halving: waves 4..7 into 0..3, 2, 3 into 0, 1, then 1 into 0).
// With one split per (b, g) the item writes the normalised output itself.
// The last item of a sequence to finish (a completion counter) sums the
// partial retrieval scores of its sequence in a fixed order and selects the
// top k, so no further launch is needed for the retrieval.
//
// Rows of more than 2048 visual tokens are selected by many workgroups
// instead (the parallel select of long_select.h, one launch after the
// attention): sum items add up the partial scores of one 2048-token chunk
// each (same fixed order) and histogram their top key digits, then the
// candidate, threshold and compaction items of the decode path run on the
// summed row.
#include "common.h"
#include "long_select.h"
#include "prefill.h"

namespace sv {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kPfStage = 32;       // keys per LDS stage (two 16-key tiles)
constexpr int kPfRowsPerWave = 32;
constexpr int kPfVPad = 32;        // bytes of padding per V row in LDS
constexpr int kPfKPad = 16;        // ... per K row (key-split path)

template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a DPP row (every lane gets it).
__device__ __forceinline__ float row16_add(float v) {
  v += dpp_row<0xB1>(v);
  v += dpp_row<0x4E>(v);
  v += dpp_row<0x141>(v);
  v += dpp_row<0x140>(v);
  return v;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int D, int W>
struct PfShape {
  static constexpr int KS = D / 32;                        // 32-wide k-steps of Q K^T
  static constexpr int DB = D / 16;                        // 16-dim blocks of P V
  static constexpr int KBYTES = 2 * KS * 1024;             // K fragments of one stage
  static constexpr int VSTR = D * 2 + kPfVPad;             // V row stride in LDS (bytes)
  static constexpr int VBYTES = kPfStage * VSTR;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int VCH = kPfStage * D / 8;             // 16-byte V chunks per stage
  static constexpr int VPT = VCH / (W * kWave);            // ... per thread
  static_assert(VCH % (W * kWave) == 0, "V stage split evenly");
};

template <int D, int W>
__global__ __launch_bounds__(W* kWave) void prefill_attn_kernel(PrefillArgs a) {
  using S = PfShape<D, W>;
  constexpr int KS = S::KS, DB = S::DB;
  __shared__ __align__(16) char lds[2 * S::BUF];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int li = lane & 15, lg = lane >> 4;
  const int C = a.CV + a.CT;

  int x = blockIdx.x;
  const int c = x % C;
  x /= C;
  const int rc = x % a.RC;
  x /= a.RC;
  const int g = x % a.Hkv;
  const int b = x / a.Hkv;

  int tl = a.txt_len ? a.txt_len[b] : 0;
  tl = tl < 0 ? 0 : (tl > a.Tmax ? a.Tmax : tl);
  const bool visual = c < a.CV;
  const int e0 = (visual ? c : c - a.CV) * a.E;
  int e1 = e0 + a.E;
  const int lim = visual ? a.N : tl;
  e1 = e1 < lim ? e1 : lim;
  const int nkeys = e1 > e0 ? e1 - e0 : 0;
  const bf16_t* kbase = visual ? a.kv + (int64_t)b * a.vbs : a.kt + (int64_t)b * a.tbs;
  const bf16_t* vbase = visual ? a.vv + (int64_t)b * a.vbs : a.vt + (int64_t)b * a.tbs;
  const int64_t ts = visual ? a.vts : a.tts;
  const int Hkv = a.Hkv;

  // Q^T fragments (B operand) of this wave's two row blocks; the text
  // position of each of this lane's rows (16 rb + li).
  bf16x8_t qf[2][KS];
  int pos[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = rc * (W * kPfRowsPerWave) + wave * kPfRowsPerWave + 16 * rb + li;
    const bool ok = row < a.rows;
    const int tau = ok ? row / a.G : 0, hh = ok ? row - tau * a.G : 0;
    pos[rb] = ok ? tl - a.Tq + tau : -1;
    const bf16_t* qr = a.q + (((int64_t)b * a.Tq + tau) * a.Hq + g * a.G + hh) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 u = ok ? *reinterpret_cast<const uint4*>(qr + 32 * s + 8 * lg) : make_uint4(0, 0, 0, 0);
      qf[rb][s] = __builtin_bit_cast(bf16x8_t, u);
    }
  }

  // Stage loads: K fragments (tile t, step s: lane (li, lg) -> key 16 t + li,
  // dims 32 s + 8 lg) directly into LDS; V rows into registers, then LDS.
  // Keys past the split read the split's first key (masked later).
  const int nst = (nkeys + kPfStage - 1) / kPfStage;
  auto key_row = [&](int k) -> int64_t { return (int64_t)(e0 + (k < nkeys ? k : 0)) * ts + g * D; };
  auto load_k = [&](int st, char* buf) {
    for (int f = wave; f < 2 * KS; f += W) {
      const int t = f / KS, s = f - t * KS;
      const bf16_t* src = kbase + key_row(st * kPfStage + 16 * t + li) + 32 * s + 8 * lg;
      char* dst = buf + f * 1024;
      __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    }
  };
  u32x4 vreg[S::VPT];
  auto load_v = [&](int st) {
#pragma unroll
    for (int i = 0; i < S::VPT; ++i) {
      const int ch = i * (W * kWave) + tid;
      const int key = ch / (D / 8), d8 = ch - key * (D / 8);
      vreg[i] = *reinterpret_cast<const u32x4*>(vbase + key_row(st * kPfStage + key) + 8 * d8);
    }
  };
  auto store_v = [&](char* buf) {
#pragma unroll
    for (int i = 0; i < S::VPT; ++i) {
      const int ch = i * (W * kWave) + tid;
      const int key = ch / (D / 8), d8 = ch - key * (D / 8);
      *reinterpret_cast<u32x4*>(buf + S::KBYTES + key * S::VSTR + d8 * 16) = vreg[i];
    }
  };

  float m[2], l[2];
  f32x4_t acc[2][DB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[rb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  float* pscore = visual ? a.pscore + ((int64_t)b * a.NP + (g * a.RC + rc) * W + wave) * a.N : nullptr;

  if (nst > 0) {
    load_k(0, lds);
    load_v(0);
    store_v(lds);
  }
  wait_stores_complete();  // direct LDS loads landed (vmcnt = 0)
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    char* cur = lds + (st & 1) * S::BUF;
    char* nxt = lds + ((st + 1) & 1) * S::BUF;
    const bool more = st + 1 < nst;
    if (more) {
      load_k(st + 1, nxt);
      load_v(st + 1);
    }
    float sck = 0.f;  // lanes li < 8: retrieval score of key 16 (li / 4) + 4 lg + li % 4
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8_t kf[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        kf[s] = *reinterpret_cast<const bf16x8_t*>(cur + ((t * KS + s) * kWave + lane) * 16);
      f32x4_t St[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[rb][s], z, 0, 0, 0);
        St[rb] = z;  // St[rb][r] = S[row 16 rb + li][key 16 t + 4 lg + r]
      }
      const int kb = st * kPfStage + 16 * t + 4 * lg;  // split-relative key of r = 0
      if (visual) {
        // Retrieval: raw logits of the key summed over this wave's rows
        // (every lane of the lane group holds each sum).
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sc = row16_add(St[0][r] + St[1][r]);
          sck = li == 4 * t + r ? sc : sck;
        }
      }
      s16x4 ph[2], pl[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float xv[4], tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int k = kb + r;
          const bool ok = k < nkeys && (visual || e0 + k <= pos[rb]);
          xv[r] = ok ? St[rb][r] * a.c2 : -INFINITY;
          tmax = fmaxf(tmax, xv[r]);
        }
        tmax = fmaxf(tmax, xor_partner<16>(tmax));
        tmax = fmaxf(tmax, xor_partner<32>(tmax));
        const float mn = fmaxf(m[rb], tmax);
        const float al = mn == -INFINITY ? 1.f : fast_exp2(m[rb] - mn);
        float p[4], ps = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = xv[r] == -INFINITY ? 0.f : fast_exp2(xv[r] - mn);
          ps += p[r];
        }
        l[rb] = l[rb] * al + ps;
        m[rb] = mn;
        // Rescale the output rows whose maximum rose (the whole wave or none).
        if (__builtin_amdgcn_ballot_w64(al != 1.f)) {
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[rb][db] *= al;
        }
        // P^T as the B operand: high bf16 part and the bf16 residual.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint16_t h = bf16_rne(p[r]);
          ph[rb][r] = (short)h;
          pl[rb][r] = (short)bf16_rne(p[r] - __uint_as_float((uint32_t)h << 16));
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        // V^T fragment: lane (li, lg) gets dim 16 db + li of keys 16 t + 4 lg .. + 3.
        const int vkey = 16 * t + 4 * lg + (li >> 2);
        const char* va = cur + S::KBYTES + vkey * S::VSTR + (16 * db + 4 * (li & 3)) * 2;
        const s16x4 vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(va));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          f32x4_t o = acc[rb][db];
          o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, ph[rb], o, 0, 0, 0);
          o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pl[rb], o, 0, 0, 0);
          acc[rb][db] = o;  // acc[rb][db][r] = O[row 16 rb + li][dim 16 db + 4 lg + r]
        }
      }
    }
    // One 128-byte store of the stage's 32 scores (lanes li < 8 of each group).
    if (visual && li < 8) {
      const int k = st * kPfStage + 16 * (li >> 2) + 4 * lg + (li & 3);
      if (k < nkeys) pscore[e0 + k] = sck;
    }
    if (more) store_v(nxt);
    wait_stores_complete();
    __syncthreads();
  }

  // Partial of split c for this wave's rows: O (unnormalised), m, l.
  float* part = a.part + (((int64_t)(b * Hkv + g) * a.RC + rc) * C + c) * (W * kPfRowsPerWave) *
                              (D + 4);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    float lt = l[rb];
    lt += xor_partner<16>(lt);
    lt += xor_partner<32>(lt);
    const int rl = wave * kPfRowsPerWave + 16 * rb + li;
    float* pr = part + (int64_t)rl * (D + 4);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<f32x4_t*>(pr + 16 * db + 4 * lg) = acc[rb][db];
    if (lg == 0) {
      pr[D] = m[rb];
      pr[D + 1] = lt;
    }
  }
}

constexpr int kPfKW = 8;  // key-split waves of the one-row-block path

// Retrieval of sequence b by one workgroup of NW waves once every partial
// score row of b is written: s[t] = sum_j pscore[b][j][t] (j = 0..NP-1 in
// order), stored to the scores row, then the top-k of the row into idx[b].
template <int NW, int KPT>
__device__ __forceinline__ void select_sequence(const PrefillArgs& a, int b, char* smem) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int N = a.N;
  const float* ps = a.pscore + (int64_t)b * a.NP * N;
  float* srow = a.scores + (int64_t)b * N;
  // The select's element layout: wave w owns [w*seg, (w+1)*seg), lane l
  // elements w*seg + 64 i + l.
  const int seg = ((N + NW * kWave - 1) / (NW * kWave)) * kWave;
  const int chunks = seg / kWave;
  const int base = wave * seg + lane;
  uint32_t key[KPT];
  if (N % 4 == 0 && chunks <= KPT && (((uintptr_t)a.scores | (uintptr_t)a.pscore) & 15) == 0) {
    // Rows of whole 16-byte groups: thread t sums keys 4t .. 4t + 3 over the
    // partial rows (one 16-byte load per row, up to 32 rows in flight, added
    // in row order as below), then the sums reach the select's element layout
    // through LDS.
    float* ssum = reinterpret_cast<float*>(smem + sizeof(SelectSmem<NW>));
    const BufRsrc rps = make_rsrc(ps, (uint32_t)((int64_t)a.NP * N * 4));
    const BufRsrc rsr = make_rsrc(srow, (uint32_t)N * 4u);
    for (int q = tid; q < N / 4; q += NW * kWave) {
      f32x4v acc = {0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < a.NP; j0 += 32) {
        f32x4v v[32];
#pragma unroll
        for (int j = 0; j < 32; ++j)
          v[j] = j0 + j < a.NP ? __builtin_bit_cast(f32x4v, __builtin_amdgcn_raw_buffer_load_b128(
                                     rps, (uint32_t)q * 16u, (uint32_t)((j0 + j) * N * 4), kCacheCoherent))
                               : f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 32; ++j)
          if (j0 + j < a.NP) acc += v[j];
      }
      store4_dev(rsr, (uint32_t)q * 16u, __builtin_bit_cast(u32x4, acc));
      *reinterpret_cast<f32x4v*>(ssum + 4 * q) = acc;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = base + i * kWave;
      key[i] = float_key(i < chunks && e < N ? ssum[e] : 0.f);
    }
    SelectSmem<NW>& sm = *reinterpret_cast<SelectSmem<NW>*>(smem);
    block_topk<NW, KPT, false, true>(nullptr, N, a.k, a.idx + (int64_t)b * a.k, sm, key);
    return;
  }
  for (int i0 = 0; i0 < chunks; i0 += KPT) {
    float sum[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) sum[i] = 0.f;
    for (int j0 = 0; j0 < a.NP; j0 += 8) {
      float v[8][KPT];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          const int e = base + (i0 + i) * kWave;
          v[j][i] = (j0 + j < a.NP && i0 + i < chunks && e < N)
                        ? load_shared_dev(ps + (int64_t)(j0 + j) * N + e) : 0.f;
        }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < KPT; ++i) sum[i] += v[j][i];
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = base + (i0 + i) * kWave;
      if (i0 + i < chunks && e < N) store_shared_dev(srow + e, sum[i]);
      if (i0 == 0) key[i] = float_key(sum[i]);
    }
  }
  SelectSmem<NW>& sm = *reinterpret_cast<SelectSmem<NW>*>(smem);
  int32_t* out = a.idx + (int64_t)b * a.k;
  if (chunks <= KPT) {
    block_topk<NW, KPT, false, true>(nullptr, N, a.k, out, sm, key);
  } else {
    wait_stores_complete();  // the row just stored is read back by the select's passes
    __syncthreads();
    block_topk<NW, KPT, true, false>(srow, N, a.k, out, sm);
  }
}

template <int D>
struct PfKwShape {
  static constexpr int KS = D / 32;                          // 32-wide k-steps of Q K^T
  static constexpr int DB = D / 16;                          // 16-dim blocks of P V
  static constexpr int VSTR = D * 2 + kPfVPad;               // V row stride in LDS (bytes)
  static constexpr int VBYTES = kPfStage * VSTR;             // one wave's V stage
  static constexpr int KSTR = D * 2 + kPfKPad;               // K row stride in LDS (bytes)
  static constexpr int KBYTES = kPfStage * KSTR;             // one wave's K stage
  static constexpr int WBYTES = VBYTES + KBYTES;             // one wave's stage buffers
  static constexpr int VPL = kPfStage * D / 8 / kWave;       // 16-byte chunks per lane (K or V)
  static constexpr int MSTR = D + 4;                         // floats per row of a merge slot
  static constexpr int MBYTES = kPfRowsPerWave * MSTR * 4;   // one merge slot (one per wave)
  static constexpr int QBYTES = 2 * KS * kWave * 16;          // Q^T fragments of the row block
  static constexpr int SBYTES = sizeof(SelectSmem<kPfKW>);
  static constexpr int MAIN0 = kPfKW * WBYTES > kPfKW * MBYTES ? kPfKW * WBYTES : kPfKW * MBYTES;
  static constexpr int MAIN = MAIN0 > SBYTES ? MAIN0 : SBYTES;  // stage buffers, merge slots, select
  static constexpr int LDS = MAIN + QBYTES;
  static constexpr int SKPT = 4;  // keys per thread kept in registers by the select (rows <= 2048)
  static_assert(VPL * kWave * 8 == kPfStage * D, "K and V stages split evenly over a wave");
  static_assert(LDS + 4 <= 160 * 1024, "one workgroup's LDS");
  static_assert(SBYTES + 2048 * 4 <= MAIN, "select state plus the summed scores of a row");
};

template <int D>
__global__ __launch_bounds__(kPfKW* kWave, 2) void prefill_attn_kw_kernel(PrefillArgs a) {
  using S = PfKwShape<D>;
  constexpr int KS = S::KS, DB = S::DB;
  __shared__ __align__(16) char lds[S::LDS];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int li = lane & 15, lg = lane >> 4;
  const int C = a.CV;

  int x = blockIdx.x;
  const int c = x % C;
  x /= C;
  const int g = x % a.Hkv;
  const int b = x / a.Hkv;

  int tl = a.txt_len ? a.txt_len[b] : 0;
  tl = tl < 0 ? 0 : (tl > a.Tmax ? a.Tmax : tl);
  const int N = a.N;
  // Keys of the sequence as one list: e < N visual tokens, N <= e < Np
  // padding (masked), e >= Np text rows e - Np; Np = N rounded up to a stage,
  // so every stage is all visual or all text.
  const int Np = (N + kPfStage - 1) / kPfStage * kPfStage;
  const int e0 = c * a.E;
  int e1 = e0 + a.E;
  e1 = e1 < Np + tl ? e1 : Np + tl;
  const int nkeys = e1 > e0 ? e1 - e0 : 0;
  const int nst = (nkeys + kPfStage - 1) / kPfStage;

  // Q^T fragments of the row block (rows li and 16 + li) in LDS, shared by
  // the waves, in the lanes' dim order (fragment (rb, s) of lane l at
  // ((rb * KS + s) * 64 + l) * 16 bytes); the text position of each of this
  // lane's rows.
  char* qbuf = lds + S::LDS - S::QBYTES;
  int pos[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = 16 * rb + li;
    const bool ok = row < a.rows;
    const int tau = ok ? row / a.G : 0, hh = ok ? row - tau * a.G : 0;
    pos[rb] = ok ? tl - a.Tq + tau : -1;
    const bf16_t* qr = a.q + (((int64_t)b * a.Tq + tau) * a.Hq + g * a.G + hh) * D + 8 * lg;
    for (int s = wave; s < KS; s += kPfKW) {
      const uint4 u = ok ? *reinterpret_cast<const uint4*>(qr + 32 * s) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(qbuf + ((rb * KS + s) * kWave + lane) * 16) = u;
    }
  }
  __syncthreads();
  auto qfrag = [&](int rb, int s) {
    return *reinterpret_cast<const bf16x8_t*>(qbuf + ((rb * KS + s) * kWave + lane) * 16);
  };

  // Each cache of (b, g) as one buffer: rows past the cache (and past the
  // text length) read as zeros, the rows of other splits are read and masked.
  const BufRsrc rkv = make_rsrc(a.kv + (int64_t)b * a.vbs + g * D,
                                (uint32_t)((int64_t)(N - 1) * a.vts * 2 + D * 2));
  const BufRsrc rvv = make_rsrc(a.vv + (int64_t)b * a.vbs + g * D,
                                (uint32_t)((int64_t)(N - 1) * a.vts * 2 + D * 2));
  const uint32_t text_ext = tl > 0 ? (uint32_t)((int64_t)(tl - 1) * a.tts * 2 + D * 2) : 0u;
  const BufRsrc rkt = make_rsrc(tl > 0 ? a.kt + (int64_t)b * a.tbs + g * D : a.kv, text_ext);
  const BufRsrc rvt = make_rsrc(tl > 0 ? a.vt + (int64_t)b * a.tbs + g * D : a.vv, text_ext);
  // K and V rows of a stage go through the wave's LDS buffers: chunk i of
  // a lane is key (64 i + lane) / (D / 8), 16 bytes at dim 8 ((64 i + lane)
  // % (D / 8)), so each load covers whole rows.  The K fragments are read
  // back from LDS (tile t, step s -> key 16 t + li, dims 32 s + 8 lg).
  constexpr int VKPI = kWave / (D / 8);  // keys per chunk index
  u32x4 kr[S::VPL];
  u32x4 vr[S::VPL];
  struct StageSrc {
    BufRsrc rk, rv;
    uint32_t rs, row0;
  };
  auto stage_src = [&](int st) {
    const int ks = e0 + st * kPfStage;  // uniform
    const bool vis = ks < Np;
    return StageSrc{vis ? rkv : rkt, vis ? rvv : rvt, (uint32_t)((vis ? a.vts : a.tts) * 2),
                    (uint32_t)(vis ? ks : ks - Np)};
  };
  auto load_k = [&](int st) {
    const StageSrc ss = stage_src(st);
    const uint32_t vo = (ss.row0 + lane / (D / 8)) * ss.rs + (lane % (D / 8)) * 16;
#pragma unroll
    for (int i = 0; i < S::VPL; ++i)
      kr[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ss.rk, vo, i * VKPI * ss.rs, kCacheStream));
  };
  auto load_v = [&](int st) {
    const StageSrc ss = stage_src(st);
    const uint32_t vo = (ss.row0 + lane / (D / 8)) * ss.rs + (lane % (D / 8)) * 16;
#pragma unroll
    for (int i = 0; i < S::VPL; ++i)
      vr[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ss.rv, vo, i * VKPI * ss.rs, kCacheStream));
  };
  char* vbuf = lds + wave * S::WBYTES;
  char* kbuf = vbuf + S::VBYTES;

  float m[2], l[2];
  f32x4_t acc[2][DB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[rb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  float* pscore = a.pscore + ((int64_t)b * a.NP + g) * N;

  if (wave < nst) {
    load_k(wave);
    load_v(wave);
  }
  for (int st = wave; st < nst; st += kPfKW) {
    // This stage's K and V rows to the wave's own LDS buffers (its reads of
    // the previous stage were issued before these writes), then the next
    // stage's loads.
    const bool more = st + kPfKW < nst;
#pragma unroll
    for (int i = 0; i < S::VPL; ++i) {
      const int ch = i * kWave + lane;
      const int key = ch / (D / 8), d8 = ch - key * (D / 8);
      *reinterpret_cast<u32x4*>(kbuf + key * S::KSTR + d8 * 16) = kr[i];
      *reinterpret_cast<u32x4*>(vbuf + key * S::VSTR + d8 * 16) = vr[i];
    }
    if (more) {
      load_k(st + kPfKW);
      load_v(st + kPfKW);
    }
    f32x4_t Sall[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kbuf + (16 * t + li) * S::KSTR +
                                                                 64 * s + 16 * lg);
          z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qfrag(rb, s), z, 0, 0, 0);
        }
        Sall[t][rb] = z;  // Sall[t][rb][r] = S[row 16 rb + li][key 16 t + 4 lg + r]
      }
    float sck = 0.f;  // lanes li < 8: retrieval score of key 16 (li / 4) + 4 lg + li % 4
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f32x4_t* St = Sall[t];
      const int kb = st * kPfStage + 16 * t + 4 * lg;  // split-relative key of r = 0
      // Retrieval: raw logits of each key summed over the row block (every
      // lane of the lane group holds each sum).
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sc = row16_add(St[0][r] + St[1][r]);
        sck = li == 4 * t + r ? sc : sck;
      }
      s16x4 ph[2], pl[2];
      float al[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float xv[4], tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int k = kb + r, e = e0 + k;
          const bool ok = k < nkeys && (e < N || (e >= Np && e - Np <= pos[rb]));
          xv[r] = ok ? St[rb][r] * a.c2 : -INFINITY;
          tmax = fmaxf(tmax, xv[r]);
        }
        tmax = fmaxf(tmax, xor_partner<16>(tmax));
        tmax = fmaxf(tmax, xor_partner<32>(tmax));
        const float mn = fmaxf(m[rb], tmax);
        al[rb] = mn == -INFINITY ? 1.f : fast_exp2(m[rb] - mn);
        float p[4], ps = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = xv[r] == -INFINITY ? 0.f : fast_exp2(xv[r] - mn);
          ps += p[r];
        }
        l[rb] = l[rb] * al[rb] + ps;
        m[rb] = mn;
        // Rescale the output rows whose maximum rose (rare after the first
        // tiles; the branch is taken by the whole wave or not at all).
        if (__builtin_amdgcn_ballot_w64(al[rb] != 1.f)) {
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[rb][db] *= al[rb];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint16_t h = bf16_rne(p[r]);
          ph[rb][r] = (short)h;
          pl[rb][r] = (short)bf16_rne(p[r] - __uint_as_float((uint32_t)h << 16));
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int vkey = 16 * t + 4 * lg + (li >> 2);
        const char* va = vbuf + vkey * S::VSTR + (16 * db + 4 * (li & 3)) * 2;
        const s16x4 vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(va));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          f32x4_t o = acc[rb][db];
          o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, ph[rb], o, 0, 0, 0);
          o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pl[rb], o, 0, 0, 0);
          acc[rb][db] = o;  // acc[rb][db][r] = O[row 16 rb + li][dim 16 db + 4 lg + r]
        }
      }
    }
    // One 128-byte store of the stage's 32 visual scores (lanes li < 8 of
    // each group; text keys and padding store nothing).
    if (li < 8) {
      const int kk = st * kPfStage + 16 * (li >> 2) + 4 * lg + (li & 3);
      if (kk < nkeys && e0 + kk < N) store_shared_dev(pscore + e0 + kk, sck);
    }
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    l[rb] += xor_partner<16>(l[rb]);
    l[rb] += xor_partner<32>(l[rb]);
  }

  // Merge the waves: slot rows [32][D + 4] = O, m, l.
  auto slot = [&](int i) { return reinterpret_cast<float*>(lds) + i * kPfRowsPerWave * S::MSTR; };
  auto put = [&](int i) {
    float* sp = slot(i);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float* pr = sp + (16 * rb + li) * S::MSTR;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4_t*>(pr + 16 * db + 4 * lg) = acc[rb][db];
      if (lg == 0) {
        pr[D] = m[rb];
        pr[D + 1] = l[rb];
      }
    }
  };
  // Every wave puts its rows in its own slot; then wave w merges rows
  // 4w .. 4w + 3 over the slots in wave order (16 lanes per row, D / 16 dims
  // per lane) and writes them.
  __syncthreads();  // every wave is past its stage buffers
  put(wave);
  __syncthreads();
  {
    constexpr int RPW = kPfRowsPerWave / kPfKW;  // rows merged per wave
    constexpr int LPR = kWave / RPW;              // lanes per row
    constexpr int DPL = D / LPR;                  // dims per lane
    static_assert(RPW * kPfKW == kPfRowsPerWave && DPL % 4 == 0, "merge split");
    const int row = wave * RPW + lane / LPR;
    const int d0 = (lane % LPR) * DPL;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPfKW; ++i) M = fmaxf(M, slot(i)[row * S::MSTR + D]);
    f32x4_t num[DPL / 4];
#pragma unroll
    for (int v = 0; v < DPL / 4; ++v) num[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
#pragma unroll
    for (int i = 0; i < kPfKW; ++i) {
      const float* pr = slot(i) + row * S::MSTR;
      const float mi = pr[D];
      const float f = mi == -INFINITY ? 0.f : fast_exp2(mi - M);
      den += pr[D + 1] * f;
#pragma unroll
      for (int v = 0; v < DPL / 4; ++v)
        num[v] += *reinterpret_cast<const f32x4_t*>(pr + d0 + 4 * v) * f;
    }
    if (C == 1) {
      // The only split: normalised output rows.
      if (row < a.rows) {
        const int tau = row / a.G, hh = row - tau * a.G;
        float* o = a.out + (((int64_t)b * a.Tq + tau) * a.Hq + g * a.G + hh) * D + d0;
        const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
        for (int v = 0; v < DPL / 4; ++v) *reinterpret_cast<f32x4_t*>(o + 4 * v) = num[v] * inv;
      }
    } else {
      float* pr = a.part + (((int64_t)(b * a.Hkv + g) * C + c) * kPfRowsPerWave + row) * (D + 4);
#pragma unroll
      for (int v = 0; v < DPL / 4; ++v) *reinterpret_cast<f32x4_t*>(pr + d0 + 4 * v) = num[v];
      if (lane % LPR == 0) {
        pr[D] = M;
        pr[D + 1] = den;
      }
    }
  }
  if (a.k <= 0 || a.long_ws) return;  // long rows: the parallel select runs after

  // The last item of sequence b: retrieval scores and the top-k.
  __shared__ uint32_t s_last;
  wait_stores_complete();  // this item's partial scores are out (device-coherent)
  __syncthreads();
  uint32_t* ctr = a.ctl + (int64_t)b * kCtrStride;
  if (tid == 0) s_last = counter_add(ctr, 1u) == (uint32_t)(a.Hkv * C) - 1 ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  select_sequence<kPfKW, S::SKPT>(a, b, lds);
  if (tid == 0) counter_reset(ctr);
}

// ---------------------------------------------------------------- long rows
// Sum item (b, p): chunk p of sequence b's scores (the element layout of
// the long-row select: p*2048 + wave*512 + 64 i + lane), stored
// device-coherent; their top 11 key bits go to a local histogram, flushed
// to replica p % kLsReps of hist1; then seq_ctr[b] += 1.
__device__ __forceinline__ void pf_sum_item(const PrefillArgs& pa, const ScanArgs& sa,
                                            const LongSelArgs& ls, int b, int p, char* smem) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int N = pa.N;
  uint32_t* lh = reinterpret_cast<uint32_t*>(smem);
  for (int i = tid; i < kLsBins; i += kItemThreads) lh[i] = 0u;
  __syncthreads();
  const float* ps = pa.pscore + (int64_t)b * pa.NP * N;
  float* srow = sa.scores + (int64_t)b * N;
  if (N % 4 == 0 && (int64_t)pa.NP * N * 4 < ((int64_t)1 << 31) &&
      (((uintptr_t)pa.pscore | (uintptr_t)sa.scores) & 15) == 0) {
    // Thread t: keys p 2048 + h 1024 + 4 t .. + 3 (h = 0, 1), one 16-byte load
    // per partial row, 16 rows in flight, added in row order.
    const BufRsrc rps = make_rsrc(ps, (uint32_t)((int64_t)pa.NP * N * 4));
    const BufRsrc rsr = make_rsrc(srow, (uint32_t)N * 4u);
    uint32_t off[2];
    f32x4v s4[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = p * kLsChunk + h * (kLsChunk / 2) + 4 * tid;
      off[h] = c < N ? (uint32_t)c * 4u : kBufOob;
      s4[h] = f32x4v{0.f, 0.f, 0.f, 0.f};
    }
    for (int j0 = 0; j0 < pa.NP; j0 += 16) {
      f32x4v v[16][2];
#pragma unroll
      for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          v[j][h] = j0 + j < pa.NP ? __builtin_bit_cast(f32x4v, __builtin_amdgcn_raw_buffer_load_b128(
                                         rps, off[h], (uint32_t)((j0 + j) * N * 4), kCacheDefault))
                                   : f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j0 + j < pa.NP) {
#pragma unroll
          for (int h = 0; h < 2; ++h) s4[h] += v[j][h];
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (off[h] == kBufOob) continue;
      store4_dev(rsr, off[h], __builtin_bit_cast(u32x4, s4[h]));
#pragma unroll
      for (int r = 0; r < 4; ++r) atomicAdd(&lh[digit1(float_key(s4[h][r]))], 1u);
    }
  } else {
    const int e0 = p * kLsChunk + wave * (kLsChunk / kItemWaves) + lane;
    float sum[kSelKpt];
#pragma unroll
    for (int i = 0; i < kSelKpt; ++i) sum[i] = 0.f;
    for (int j0 = 0; j0 < pa.NP; j0 += 4) {
      float v[4][kSelKpt];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < kSelKpt; ++i) {
          const int e = e0 + i * kWave;
          v[j][i] = (j0 + j < pa.NP && e < N) ? ps[(int64_t)(j0 + j) * N + e] : 0.f;
        }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < kSelKpt; ++i) sum[i] += v[j][i];
    }
#pragma unroll
    for (int i = 0; i < kSelKpt; ++i) {
      const int e = e0 + i * kWave;
      if (e < N) {
        store_shared_dev(srow + e, sum[i]);
        atomicAdd(&lh[digit1(float_key(sum[i]))], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* gh = ls.hist1 + ((int64_t)b * kLsReps + (p & (kLsReps - 1))) * kLsBins;
  for (int i = tid; i < kLsBins; i += kItemThreads) {
    const uint32_t v = lh[i];
    if (v) __hip_atomic_fetch_add(gh + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wait_stores_complete();
  __syncthreads();
  if (tid == 0) counter_add(&sa.seq_ctr[b * kCtrStride], 1u);
}

// Items in phase order: B*P sum items, B*P candidate items, B threshold
// items, B*P compaction items (each waits only on items before it).
__global__ __launch_bounds__(kItemThreads) void prefill_long_select_kernel(PrefillArgs pa,
                                                                           ScanArgs sa,
                                                                           LongSelArgs ls) {
  extern __shared__ __align__(16) char smem[];
  const uint32_t B = (uint32_t)pa.B, P = (uint32_t)ls.P;
  uint32_t u = blockIdx.x;
  if (u < B * P) {
    pf_sum_item(pa, sa, ls, u / P, u % P, smem);
  } else if ((u -= B * P) < B * P) {
    cand_item(sa, ls, u / P, u % P, smem);
  } else if ((u -= B * P) < B) {
    thr_item(sa, ls, u, smem);
  } else {
    u -= B;
    compact_item(sa, ls, u / P, u % P, smem);
  }
}

hipError_t launch_prefill_long_select(const PrefillArgs& a, hipStream_t st) {
  const int P = (a.N + kLsChunk - 1) / kLsChunk;
  char* w = static_cast<char*>(a.long_ws);
  auto take = [&](size_t n) {
    char* r = w;
    w += (n + 255) & ~(size_t)255;
    return r;
  };
  LongSelArgs ls{};
  ls.P = P;
  ls.readers = (uint32_t)P;  // the compaction items read the threshold
  ls.ctl = reinterpret_cast<uint32_t*>(take((size_t)a.B * kLsCtlLines * kCtrStride * 4));
  ls.hist1 = reinterpret_cast<uint32_t*>(take((size_t)a.B * kLsReps * kLsBins * 4));
  ls.hist2 = reinterpret_cast<uint32_t*>(take((size_t)a.B * kLsBins * 4));
  ls.cand = reinterpret_cast<uint64_t*>(take((size_t)a.B * kLsCandCap * 8));
  ls.chunk_hi = reinterpret_cast<uint32_t*>(take((size_t)a.B * P * 4));
  ls.offs = reinterpret_cast<uint32_t*>(take((size_t)a.B * P * 4));
  ScanArgs sa{};
  sa.N = a.N;
  sa.k = a.k;
  sa.idx = a.idx;
  sa.scores = a.scores;
  sa.items_per_seq = P;
  sa.seq_ctr = a.ctl + (size_t)a.B * kCtrStride;
  sa.hist1 = ls.hist1;
  sa.spin_limit = kSpinLimit;
  size_t lds = (size_t)kLsBins * 4;
  if (cand_smem_bytes() > lds) lds = cand_smem_bytes();
  if (thr_smem_bytes(P) > lds) lds = thr_smem_bytes(P);
  if (sizeof(SelectSmem<kItemWaves>) > lds) lds = sizeof(SelectSmem<kItemWaves>);
  const unsigned items = (unsigned)(3 * a.B * P + a.B);
  hipLaunchKernelGGL(prefill_long_select_kernel, dim3(items), dim3(kItemThreads), lds, st, a, sa, ls);
  return hipGetLastError();
}

// Merge the C splits of every row: out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
template <int D>
__global__ __launch_bounds__(D) void prefill_combine_kernel(PrefillArgs a) {
  const int RCH = a.W * kPfRowsPerWave;
  int x = blockIdx.x;
  const int rl = x % RCH;
  x /= RCH;
  const int rc = x % a.RC;
  x /= a.RC;
  const int g = x % a.Hkv;
  const int b = x / a.Hkv;
  const int row = rc * RCH + rl;
  if (row >= a.rows) return;
  const int C = a.CV + a.CT;
  const float* p = a.part + ((int64_t)(b * a.Hkv + g) * a.RC + rc) * C * RCH * (D + 4) +
                   (int64_t)rl * (D + 4);
  const int64_t cs = (int64_t)RCH * (D + 4);
  const int d = threadIdx.x;
  // Batches of up to kCh splits: their (m, l) pairs go to LDS in one round
  // trip, then every thread adds its dim of 16 splits per round trip; the
  // running maximum rescales the sums between batches.
  constexpr int kCh = 128;
  __shared__ float s_m[kCh], s_l[kCh];
  float M = -INFINITY, num = 0.f, den = 0.f;
  for (int c0 = 0; c0 < C; c0 += kCh) {
    const int n = C - c0 < kCh ? C - c0 : kCh;
    __syncthreads();  // the previous batch is read
    for (int j = d; j < n; j += D) {
      s_m[j] = p[(c0 + j) * cs + D];
      s_l[j] = p[(c0 + j) * cs + D + 1];
    }
    __syncthreads();
    float bm = -INFINITY;
    for (int j = 0; j < n; ++j) bm = fmaxf(bm, s_m[j]);
    const float mn = fmaxf(M, bm);
    const float sc = M == -INFINITY ? 0.f : fast_exp2(M - mn);
    num *= sc;
    den *= sc;
    M = mn;
    for (int j0 = 0; j0 < n; j0 += 16) {
      float ov[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) ov[j] = j0 + j < n ? p[(c0 + j0 + j) * cs + d] : 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j0 + j < n) {
          const float mc = s_m[j0 + j];
          const float w = mc == -INFINITY ? 0.f : fast_exp2(mc - M);
          num = fmaf(w, ov[j], num);
          den = fmaf(w, s_l[j0 + j], den);
        }
      }
    }
  }
  const int tau = row / a.G, hh = row - tau * a.G;
  a.out[(((int64_t)b * a.Tq + tau) * a.Hq + g * a.G + hh) * D + d] = den > 0.f ? num / den : 0.f;
}

// scores[b][t] = sum over the NP partials (fixed order).
__global__ __launch_bounds__(256) void prefill_scores_kernel(PrefillArgs a, float* scores) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.B * a.N) return;
  const int b = (int)(i / a.N), t = (int)(i - (int64_t)b * a.N);
  const float* p = a.pscore + (int64_t)b * a.NP * a.N + t;
  float s = 0.f;
  for (int j0 = 0; j0 < a.NP; j0 += 8) {  // batches of 8 loads in flight, summed in order
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = j0 + j < a.NP ? p[(int64_t)(j0 + j) * a.N] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += v[j];
  }
  scores[i] = s;
}

template <int D>
hipError_t prefill_go(const PrefillArgs& a, hipStream_t st) {
  const int64_t items = (int64_t)a.B * a.Hkv * a.RC * (a.CV + a.CT);
  if (a.KW > 1) {
    hipLaunchKernelGGL((prefill_attn_kw_kernel<D>), dim3((unsigned)items), dim3(kPfKW * kWave), 0,
                       st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.CV + a.CT == 1) return e;
    const int64_t rows = (int64_t)a.B * a.Hkv * kPfRowsPerWave;
    hipLaunchKernelGGL((prefill_combine_kernel<D>), dim3((unsigned)rows), dim3(D), 0, st, a);
    return hipGetLastError();
  }
  if (a.W == 2)
    hipLaunchKernelGGL((prefill_attn_kernel<D, 2>), dim3((unsigned)items), dim3(2 * kWave), 0, st, a);
  else if (a.W == 4)
    hipLaunchKernelGGL((prefill_attn_kernel<D, 4>), dim3((unsigned)items), dim3(4 * kWave), 0, st, a);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.B * a.Hkv * a.RC * a.W * kPfRowsPerWave;
  hipLaunchKernelGGL((prefill_combine_kernel<D>), dim3((unsigned)rows), dim3(D), 0, st, a);
  return hipGetLastError();
}

}  // namespace

PrefillPlan prefill_plan(int B, int Tq, int Hq, int Hkv, int N, int Tmax) {
  PrefillPlan p{};
  p.rows = Tq * (Hq / Hkv);
  if (p.rows <= kPfRowsPerWave) {
    // About 256 items (one per compute unit), splits of whole stages per wave.
    p.W = 1;
    p.RC = 1;
    p.KW = kPfKW;
    const int64_t heads = (int64_t)B * Hkv;
    int64_t C = (256 + heads / 2) / heads;
    if (C < 1) C = 1;
    const int64_t tot = ((int64_t)N + kPfStage - 1) / kPfStage * kPfStage + Tmax;  // visual keys padded to a stage, then text
    const int64_t unit = (int64_t)kPfKW * kPfStage;
    int64_t E = (tot + C - 1) / C;
    E = (E + unit - 1) / unit * unit;
    p.E = (int)E;
    p.CV = (int)((tot + E - 1) / E);
    p.CT = 0;
    p.NP = Hkv;
    return p;
  }
  p.KW = 1;
  p.W = p.rows <= 64 ? 2 : 4;
  p.RC = (p.rows + p.W * kPfRowsPerWave - 1) / (p.W * kPfRowsPerWave);
  // At most about 512 items (two per compute unit at this kernel's
  // occupancy) so that they run in one round: a second, nearly empty round
  // would double the time.
  const int64_t heads = (int64_t)B * Hkv * p.RC;
  const int64_t cmax = heads >= 256 ? 2 : 512 / heads;
  int64_t E = ((int64_t)N + Tmax + cmax - 2) / (cmax > 2 ? cmax - 1 : 1);
  E = (E + kPfStage - 1) / kPfStage * kPfStage;
  if (E < 64) E = 64;
  while (((int64_t)N + E - 1) / E + ((int64_t)Tmax + E - 1) / E > cmax && E < (int64_t)N + Tmax)
    E += kPfStage;
  p.E = (int)E;
  p.CV = (int)((N + E - 1) / E);
  p.CT = (int)((Tmax + E - 1) / E);
  p.NP = Hkv * p.RC * p.W;
  return p;
}

size_t prefill_long_select_bytes(int B, int N) {
  if (N <= kItemThreads * kSelKpt) return 0;
  const size_t P = (size_t)(N + kLsChunk - 1) / kLsChunk;
  auto al = [](size_t n) { return (n + 255) & ~(size_t)255; };
  return al((size_t)B * kLsCtlLines * kCtrStride * 4) + al((size_t)B * kLsReps * kLsBins * 4) +
         al((size_t)B * kLsBins * 4) + al((size_t)B * kLsCandCap * 8) + 2 * al((size_t)B * P * 4);
}

size_t prefill_part_floats(int B, int Hkv, int D, const PrefillPlan& p) {
  return (size_t)B * Hkv * p.RC * (p.CV + p.CT) * p.W * kPfRowsPerWave * (D + 4);
}

hipError_t launch_prefill(const PrefillArgs& a, float* scores, int k, int32_t* idx,
                          hipStream_t st) {
  hipError_t e = a.D == 128 ? prefill_go<128>(a, st) : prefill_go<64>(a, st);
  if (e != hipSuccess) return e;
  if (a.long_ws) return k > 0 ? launch_prefill_long_select(a, st) : hipSuccess;
  if (a.KW > 1) return e;  // the key-split path selects in the attention launch
  const int64_t n = (int64_t)a.B * a.N;
  hipLaunchKernelGGL(prefill_scores_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a,
                     scores);
  e = hipGetLastError();
  if (e != hipSuccess || k <= 0) return e;
  return launch_topk_rows(scores, a.B, a.N, a.N, k, idx, st);
}

}  // namespace sv
