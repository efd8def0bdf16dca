// Shared device helpers and the internal launcher interface of libsv.
// Internal header: not part of the C ABI (that is include/sv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;

// ---------------------------------------------------------------- dtypes
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- buffer loads
// A raw buffer resource (base, byte extent) lives in scalar registers; a load
// takes a 32-bit per-lane byte offset plus a wave-uniform byte offset, and
// any access at or past the extent returns zero without touching memory.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
constexpr uint32_t kBufOob = 0x80000000u;  // an offset past every extent in use
constexpr int kCacheStream = 2;            // non-temporal: data read once
constexpr int kCacheDefault = 0;

__device__ __forceinline__ BufRsrc make_rsrc(const void* base, uint32_t extent_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)extent_bytes,
                                           0x00020000);
}

// 16-byte vector of storage elements, widened to fp32.
template <typename T> struct Vec;

template <> struct Vec<bf16_t> {
  static constexpr int kElems = 8;
  u32x4 raw;
  __device__ __forceinline__ void load(const bf16_t* p) { raw = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void load_stream(const bf16_t* p) {
    raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  template <int Aux>
  __device__ __forceinline__ void load_buf(BufRsrc r, uint32_t voff, uint32_t soff) {
    raw = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, Aux));
  }
  __device__ __forceinline__ void zero() { raw = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void to_f32(float* f) const {
    f[0] = bf16_lo(raw.x); f[1] = bf16_hi(raw.x);
    f[2] = bf16_lo(raw.y); f[3] = bf16_hi(raw.y);
    f[4] = bf16_lo(raw.z); f[5] = bf16_hi(raw.z);
    f[6] = bf16_lo(raw.w); f[7] = bf16_hi(raw.w);
  }
};

template <> struct Vec<float> {
  static constexpr int kElems = 4;
  f32x4v raw;
  __device__ __forceinline__ void load(const float* p) { raw = *reinterpret_cast<const f32x4v*>(p); }
  __device__ __forceinline__ void load_stream(const float* p) {
    raw = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
  }
  template <int Aux>
  __device__ __forceinline__ void load_buf(BufRsrc r, uint32_t voff, uint32_t soff) {
    raw = __builtin_bit_cast(f32x4v, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, Aux));
  }
  __device__ __forceinline__ void zero() { raw = f32x4v{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void to_f32(float* f) const {
    f[0] = raw.x; f[1] = raw.y; f[2] = raw.z; f[3] = raw.w;
  }
};

// ---------------------------------------------------------------- keys
// Order-preserving map fp32 -> uint32 (larger float -> larger key).  -0.0 is
// canonicalised to +0.0 so that equal values compare equal.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of float_key (for keys of finite or infinite values).
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---------------------------------------------------------------- reductions
template <int Width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < Width; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

template <int Width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < Width; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over aligned groups of Width lanes (a power of two up to 64), the total
// in every lane of the group.  Inside a 16-lane row the steps are DPP moves
// (quad xor 1, quad xor 2, half-row mirror, row mirror: VALU, no LDS trip);
// wider groups add cross-row shuffles.  Every lane adds the same two partial
// sums at each step, so all lanes of a group get bit-identical totals, equal
// to the xor-butterfly's.
// The value of lane (lane ^ OFF), OFF a power of two below 64, without an
// LDS trip: a DPP row rotation for 8; for 16 and 32 the row-swap moves
// (v_permlane16_swap / v_permlane32_swap) applied to v and itself return
// both halves of each pair, and the lane keeps the other one.
template <int OFF>
__device__ __forceinline__ float xor_partner(float v) {
  const int lane = threadIdx.x & (kWave - 1);
  if constexpr (OFF == 8) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  } else if constexpr (OFF == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  } else {
    return __shfl_xor(v, OFF, kWave);
  }
}

template <int Width>
__device__ __forceinline__ float lane_group_sum(float v) {
#define SV_DPP_ADD(ctrl) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xf, 0xf, false))
  if constexpr (Width >= 2) SV_DPP_ADD(0xB1);   // quad_perm [1,0,3,2]
  if constexpr (Width >= 4) SV_DPP_ADD(0x4E);   // quad_perm [2,3,0,1]
  if constexpr (Width >= 8) SV_DPP_ADD(0x141);  // row_half_mirror
  if constexpr (Width >= 16) SV_DPP_ADD(0x140); // row_mirror
#undef SV_DPP_ADD
  if constexpr (Width >= 32) v += xor_partner<16>(v);
  if constexpr (Width >= 64) v += xor_partner<32>(v);
  return v;
}

// Whole-wave inclusive prefix sum (all 64 lanes active), DPP only: row
// shifts build 16-lane scans, then row broadcasts carry the row totals.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Whole-wave min and max (all 64 lanes active), returned wave-uniform:
// butterflies inside each 16-lane row, then the four row results.
__device__ __forceinline__ void wave_minmax(float& mn, float& mx) {
#define SV_DPP_F(x, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xf, 0xf, false))
  mn = fminf(mn, SV_DPP_F(mn, 0xB1));   // quad_perm [1,0,3,2]
  mx = fmaxf(mx, SV_DPP_F(mx, 0xB1));
  mn = fminf(mn, SV_DPP_F(mn, 0x4E));   // quad_perm [2,3,0,1]
  mx = fmaxf(mx, SV_DPP_F(mx, 0x4E));
  mn = fminf(mn, SV_DPP_F(mn, 0x141));  // row_half_mirror
  mx = fmaxf(mx, SV_DPP_F(mx, 0x141));
  mn = fminf(mn, SV_DPP_F(mn, 0x140));  // row_mirror
  mx = fmaxf(mx, SV_DPP_F(mx, 0x140));
#undef SV_DPP_F
  float a = mn, b = mx;
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    a = fminf(a, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mn), r)));
    b = fmaxf(b, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), r)));
  }
  mn = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a)));
  mx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(b)));
}

// ---------------------------------------------------------------- cross-workgroup hand-off
// Each XCD has its own L2, and an agent-scope fence would write back or
// invalidate a whole L2.  Data handed from one workgroup to another inside a
// kernel therefore goes through agent-scope relaxed atomic stores and loads
// (coherent at device scope, no cache maintenance); the writer waits for its
// stores to complete (vmcnt = 0) before its workgroup bumps the counter.
__device__ __forceinline__ void store_shared_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_shared_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_complete() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt/lgkmcnt unconstrained
}
__device__ __forceinline__ int32_t load_shared_dev_i32(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_flag(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_flag(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t counter_add(uint32_t* c, uint32_t v) {
  return __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void counter_reset(uint32_t* c) {
  __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Agent-coherent 4- and 16-byte buffer accesses (sc1: served past the
// XCD-local L2, like the agent-scope atomic loads and stores above).
constexpr int kCacheCoherent = 16;
__device__ __forceinline__ uint32_t load1_dev(BufRsrc r, uint32_t voff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, kCacheCoherent);
}
__device__ __forceinline__ u32x4 load4_dev(BufRsrc r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kCacheCoherent));
}
__device__ __forceinline__ void store4_dev(BufRsrc r, uint32_t voff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, kCacheCoherent);
}

// Counters and flags touched by many workgroups each sit on their own
// 128-byte line: same-line atomics from many workgroups serialise.
constexpr int kCtrStride = 32;  // uint32 words

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are already validated.

// Default bound of every in-kernel wait, in polls (a few seconds of polling;
// every awaited item is dispatched before its waiter, so no wait comes near it).
constexpr uint32_t kSpinLimit = 1u << 24;

// Compute units of the current device.
int device_cu_count();

// Scan rows per work item when the caller does not choose (0).
int scan_rows_per_item(int B, int N, int LPR, int nseg);
// Rows per item for at most about target_items items in all.
int scan_rows_for_items(int B, int N, int LPR, int nseg, long target_items);

hipError_t launch_retrieve(const void* q, int B, int Tq, int Hq, const void* kv, int64_t bstride,
                           int64_t tstride, int N, int Hkv, int D, int dtype, float* scores, int k,
                           int32_t* idx_out, uint32_t* counters, int rows_per_item,
                           hipStream_t stream);

hipError_t launch_topk_rows(const float* vals, int rows, int64_t row_stride, int N, int k,
                            int32_t* out, hipStream_t stream);

// One split's partial result of one query head: acc[D], m, l, two pad
// words (rows stay 16-byte aligned for the combine's vector loads).
__host__ __device__ constexpr int attn_part_stride(int D) { return D + 4; }

// Split plan of the decode attention: EPL entries per lane, SE entries per
// split, CT text splits then CV visual splits.
struct AttnPlan {
  int EPL, SE, CT, CV;
};
constexpr long kAttnTargetItems = 2048;       // standalone attention launch
constexpr long kFusedAttnTargetItems = 2048;  // fused layer: smaller splits start sooner
AttnPlan attn_plan(int B, int Hkv, int D, int VE, int k, int Tmax, long target_items);
// The fused launch's plan: attn_plan with kFusedAttnTargetItems, 4 or 8 entries per lane.
AttnPlan fused_attn_plan(int B, int Hkv, int D, int VE, int k, int Tmax, int N);
// Fused launch over rows longer than one select chunk (2048 scores) with few
// (sequence, KV head, chunk) triples: the visual attention runs chunk by
// chunk, one split per chunk, and starts before the threshold is known.
bool fused_chunk_attn(int B, int Hkv, int N, int k);

hipError_t launch_attn(const void* q, int B, int Hq, const void* kv, const void* vv,
                       int64_t vbs, int64_t vts, int N, int Hkv, int D, const int32_t* idx,
                       int k, const void* kt, const void* vt, int64_t tbs, int64_t tts,
                       const int32_t* txt_len, int Tmax, int dtype, float scale, float* out,
                       float* partials, uint32_t* counters, int epl, hipStream_t stream);

// Retrieval + sparse attention of one layer in one launch (Tq = 1).
struct FusedLaunch {
  const void* q;
  int B, Hq, Hkv, D, dtype;
  const void* k_vis;
  const void* v_vis;
  int64_t vbs, vts;
  int N, k;
  const void* k_txt;
  const void* v_txt;
  int64_t tbs, tts;
  const int32_t* txt_len;
  int Tmax;
  float scale;
  int32_t* idx;        // [B][k]
  float* scores_ws;    // [B][N] in the workspace, zero before the launch
  float* scores_out;   // [B][N] caller's copy of the scores, may be null
  float* out;          // [B][Hq][D]
  float* part;         // partials
  // Control words, each on its own 128-byte line (stride 32 words), zero
  // before the launch and zero again after it.
  uint32_t* seq_ctr;   // [B]
  uint32_t* ready;     // [B]
  uint32_t* vis_done;  // [B]
  uint32_t* comb_ctr;  // [B][Hkv]
  uint32_t* idx_enc;   // [B][k] zero before the launch and after it
  // Rows longer than the single-workgroup select: long_select_bytes(B, N)
  // bytes whose first long_select_zero_bytes(B) are zero before the launch
  // and zero again after it.
  void* long_ws;
  int Tq;              // query tokens summed by the scan (0: 1)
  // Scan and select only (sv_retrieve on rows longer than the single-
  // workgroup select): no attention items; ready and idx_enc are unused.
  bool retrieve_only;
  int rows_per_item;   // 0: default
  int epl;             // 0: default
  uint32_t spin_limit; // polls before an in-kernel wait gives up (0: kSpinLimit)
  uint32_t* status;    // sticky status word: give-up bits are ORed in (may be null)
};
hipError_t launch_fused(const FusedLaunch& f, hipStream_t stream);
size_t long_select_bytes(int B, int N);  // 0 when rows take the single-workgroup select
size_t long_select_zero_bytes(int B, int N);

bool salience_supported(int N, int D);

// colsum_ws [F*H][N], redo_ws [F*H], lse_ws [F*H][N] (used by the two-pass
// streaming kernels for frames beyond the on-chip kernels), sal [F][N].
hipError_t launch_salience(const void* q, const void* k, int F, int H, int N, int D,
                           float scale, float* colsum_ws, int32_t* redo_ws, float* lse_ws,
                           float* sal, hipStream_t stream);

// Two streaming passes for any N (8 <= D <= 128, D % 8 == 0): per-row lse,
// then column sums; c2 = scale * log2(e).
bool salience_stream_supported(int N, int D);
hipError_t launch_salience_stream(const void* q, const void* k, int FH, int N, int D, float c2,
                                  float* lse_ws, float* colsum_ws, hipStream_t stream);

}  // namespace sv
