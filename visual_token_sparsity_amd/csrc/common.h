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

// 16-byte vector of storage elements, widened to fp32.
template <typename T> struct Vec;

template <> struct Vec<bf16_t> {
  static constexpr int kElems = 8;
  u32x4 raw;
  __device__ __forceinline__ void load(const bf16_t* p) { raw = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void load_stream(const bf16_t* p) {
    raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
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
__device__ __forceinline__ uint32_t counter_add(uint32_t* c, uint32_t v) {
  return __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void counter_reset(uint32_t* c) {
  __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are already validated.
hipError_t launch_retrieve(const void* q, int B, int Tq, int Hq, const void* kv, int64_t bstride,
                           int64_t tstride, int N, int Hkv, int D, int dtype, float* scores, int k,
                           int32_t* idx_out, uint32_t* counters, hipStream_t stream);

hipError_t launch_topk_rows(const float* vals, int rows, int64_t row_stride, int N, int k,
                            int32_t* out, hipStream_t stream);

int attn_splits(int B, int Hkv, int D, int dtype, int k, int Tmax, int* epl_out);

hipError_t launch_attn(const void* q, int B, int Hq, const void* kv, const void* vv,
                       int64_t vbs, int64_t vts, int N, int Hkv, int D, const int32_t* idx,
                       int k, const void* kt, const void* vt, int64_t tbs, int64_t tts,
                       const int32_t* txt_len, int Tmax, int dtype, float scale, float* out,
                       float* partials, uint32_t* counters, hipStream_t stream);

bool salience_supported(int N, int D);

hipError_t launch_salience(const void* q, const void* k, int F, int H, int N, int D,
                           float scale, float* colsum_ws, float* sal, hipStream_t stream);

}  // namespace sv
