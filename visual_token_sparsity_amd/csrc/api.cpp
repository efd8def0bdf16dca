// C ABI of libsv (declared in include/sv.h): argument validation, workspace
// carving and kernel launches.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "common.h"
#include "pack.h"
#include "prefill.h"
#include "summary.h"
#include "sv.h"

namespace {

thread_local std::string g_err;

sv_status fail(sv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

sv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SV_OK;
  return fail(SV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int vec_elems(sv_dtype dt) { return dt == SV_BF16 ? 8 : 4; }

bool dtype_ok(sv_dtype dt) { return dt == SV_BF16 || dt == SV_F32; }

// Polls before an in-kernel wait gives up (sv_set_wait_limit).
std::atomic<uint32_t> g_wait_limit{sv::kSpinLimit};

// Workspaces whose kernels wait on each other start with one 256-byte status
// line; its first word collects the give-up bits of those waits.
constexpr size_t kStatusBytes = 256;

// The kernels address one sequence's cache slice (rows 0..n-1 at `tstride`
// elements apart, each `row` elements long) with 32-bit byte offsets.
bool extent_ok(int64_t n, int64_t tstride, int64_t row, sv_dtype dt) {
  if (n <= 0) return true;
  const int64_t es = dt == SV_BF16 ? 2 : 4;
  return ((n - 1) * tstride + row) * es < ((int64_t)1 << 31);
}

}  // namespace

namespace sv {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace sv

// ---------------------------------------------------------------- static scratch
// Workspace of sv_retrieve_attend_noalloc: SV_NOALLOC_SCRATCH_BYTES per device,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in; only the address hipGetSymbolAddress returns (per device) is used.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Zero n16 16-byte words (a kernel rather than a memset node, so the call
// can be captured in a HIP graph).
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The device address of the current device's scratch (looked up on its
// first use on that device, with the device current).
sv_status scratch_ptr(void** out, const char* fn) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SV_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SV_EUNSUPPORTED, "%s: device %d beyond the %d supported", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess || !p)
      return fail(SV_EHIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(g));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SV_OK;
}

}  // namespace

// The static scratch as the workspace of one call: at most
// SV_NOALLOC_SCRATCH_BYTES, its first `need` bytes zeroed on the stream (the
// control words, index copy and status line must start at zero; the array
// keeps whatever the previous call left).
static sv_status scratch_workspace(size_t need, hipStream_t st, void** ws, const char* fn) {
  if (need > (size_t)SV_NOALLOC_SCRATCH_BYTES)
    return fail(SV_EWORKSPACE, "%s: needs %zu bytes of scratch, more than the %zu-byte static scratch",
                fn, need, (size_t)SV_NOALLOC_SCRATCH_BYTES);
  const sv_status s = scratch_ptr(ws, fn);
  if (s != SV_OK) return s;
  const size_t n16 = (need + 15) / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (uint4*)*ws, n16);
  return hip_status(hipGetLastError(), fn);
}

extern "C" {

int sv_version(void) { return 120; }

const char* sv_last_error(void) { return g_err.c_str(); }

uint32_t sv_set_wait_limit(uint32_t polls) {
  return g_wait_limit.exchange(polls ? polls : sv::kSpinLimit);
}

sv_status sv_workspace_status(const void* workspace, void* stream) {
  if (!workspace) {
    // The static scratch of the current device (sv_retrieve_attend_noalloc).
    void* p = nullptr;
    const sv_status s = scratch_ptr(&p, "sv_workspace_status");
    if (s != SV_OK) return s;
    workspace = p;
  }
  uint32_t word = 0;
  hipStream_t st = (hipStream_t)stream;
  sv_status s = hip_status(hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, st),
                           "sv_workspace_status copy");
  if (s != SV_OK) return s;
  s = hip_status(hipStreamSynchronize(st), "sv_workspace_status sync");
  if (s != SV_OK) return s;
  if (word == 0) return SV_OK;
  return fail(SV_EHIP,
              "sv_workspace_status: an in-kernel wait gave up (bits 0x%x: 1 scores, 2 indices, "
              "4 scan count, 8 candidate count, 16 threshold); outputs of the calls on this "
              "workspace since it was zeroed are invalid: zero it before reuse",
              word);
}

// ---------------------------------------------------------------- retrieval
// Workspace of sv_retrieve: [status line][scores B*N fp32][counters B lines]
// and, for rows longer than the single-workgroup select, the long-row select
// workspace.
static size_t retrieve_scores_bytes(int B, int N) { return align256((size_t)B * (size_t)N * sizeof(float)); }

// Control words: one 128-byte line each.
static size_t ctr_bytes(size_t n) { return align256(n * sv::kCtrStride * sizeof(uint32_t)); }

size_t sv_retrieve_workspace(int B, int N, int k) {
  (void)k;
  if (B < 1 || N < 1) return kStatusBytes;
  return kStatusBytes + retrieve_scores_bytes(B, N) + ctr_bytes((size_t)B) +
         sv::long_select_bytes(B, N);
}

sv_status sv_retrieve(const void* q, int B, int Tq, int Hq, const void* k_vis, int64_t k_bstride,
                      int64_t k_tstride, int N, int Hkv, int D, sv_dtype dtype, int k,
                      int32_t* idx_out, float* scores_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!q || !k_vis || !workspace) return fail(SV_EINVAL, "sv_retrieve: NULL q, k_vis or workspace");
  if (B < 1 || B > 65535 || Tq < 1 || Hq < 1 || Hkv < 1 || N < 1)
    return fail(SV_EINVAL, "sv_retrieve: bad sizes B=%d Tq=%d Hq=%d Hkv=%d N=%d", B, Tq, Hq, Hkv, N);
  if (k < 0 || k > N) return fail(SV_EINVAL, "sv_retrieve: k=%d outside [0, N=%d]", k, N);
  if (k > 0 && !idx_out) return fail(SV_EINVAL, "sv_retrieve: NULL idx_out");
  if (Hq % Hkv) return fail(SV_EINVAL, "sv_retrieve: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (!dtype_ok(dtype)) return fail(SV_EUNSUPPORTED, "sv_retrieve: dtype %d", (int)dtype);
  if (D != 64 && D != 128) return fail(SV_EUNSUPPORTED, "sv_retrieve: D=%d (64 or 128)", D);
  if (Hq / Hkv > 64) return fail(SV_EUNSUPPORTED, "sv_retrieve: group size %d > 64", Hq / Hkv);
  const int64_t R = (int64_t)Hkv * D;
  if (R > (dtype == SV_BF16 ? 8192 : 4096))
    return fail(SV_EUNSUPPORTED, "sv_retrieve: row Hkv*D=%lld too long", (long long)R);
  const int ve = vec_elems(dtype);
  if (k_tstride < R || k_bstride < 0 || k_tstride % ve || k_bstride % ve)
    return fail(SV_EINVAL, "sv_retrieve: strides (%lld, %lld) must be >= row and multiples of %d",
                (long long)k_bstride, (long long)k_tstride, ve);
  if (!aligned16(q) || !aligned16(k_vis))
    return fail(SV_EINVAL, "sv_retrieve: q and k_vis must be 16-byte aligned");
  if (!extent_ok(N, k_tstride, R, dtype))
    return fail(SV_EUNSUPPORTED, "sv_retrieve: one sequence's key slice spans 2 GiB or more");
  if (workspace_bytes < sv_retrieve_workspace(B, N, k))
    return fail(SV_EWORKSPACE, "sv_retrieve: workspace %zu < %zu bytes", workspace_bytes,
                sv_retrieve_workspace(B, N, k));
  uint32_t* status = (uint32_t*)workspace;
  char* ws = (char*)workspace + kStatusBytes;
  float* scores = scores_out ? scores_out : (float*)ws;
  uint32_t* counters = (uint32_t*)(ws + retrieve_scores_bytes(B, N));
  if (k > 0 && sv::long_select_bytes(B, N) > 0 && Hq / Hkv <= 8) {
    // Long rows: the scan and the parallel select of the one-launch layer
    // (every pass over a row split into 2048-score chunks), no attention.
    sv::FusedLaunch f{};
    f.q = q;
    f.B = B;
    f.Tq = Tq;
    f.Hq = Hq;
    f.Hkv = Hkv;
    f.D = D;
    f.dtype = (int)dtype;
    f.k_vis = k_vis;
    f.v_vis = k_vis;
    f.vbs = k_bstride;
    f.vts = k_tstride;
    f.N = N;
    f.k = k;
    f.scale = 1.0f;
    f.idx = idx_out;
    f.scores_ws = (float*)ws;
    f.scores_out = scores_out;
    f.seq_ctr = counters;
    f.long_ws = (char*)counters + ctr_bytes((size_t)B);
    f.retrieve_only = true;
    f.spin_limit = g_wait_limit.load(std::memory_order_relaxed);
    f.status = status;
    return hip_status(sv::launch_fused(f, (hipStream_t)stream), "sv_retrieve");
  }
  return hip_status(sv::launch_retrieve(q, B, Tq, Hq, k_vis, k_bstride, k_tstride, N, Hkv, D,
                                        (int)dtype, scores, k, idx_out, counters, 0,
                                        (hipStream_t)stream),
                    "sv_retrieve");
}

// ---------------------------------------------------------------- attention
// Workspace of sv_sparse_decode_attn: [partials B*Hq*C*(D+4) fp32][counters B*Hkv uint32].
static size_t attn_partial_bytes(int B, int Hq, int Hkv, int D, int k, int Tmax,
                                 bool fused = false, int N = 0) {
  size_t best = 0;
  for (int ve = 4; ve <= 8; ve += 4) {
    const sv::AttnPlan p = fused ? sv::fused_attn_plan(B, Hkv, D, ve, k, Tmax, N)
                                 : sv::attn_plan(B, Hkv, D, ve, k, Tmax, sv::kAttnTargetItems);
    const size_t bytes = (size_t)B * Hq * (p.CT + p.CV) * sv::attn_part_stride(D) * sizeof(float);
    if (bytes > best) best = bytes;
  }
  return align256(best);
}

size_t sv_sparse_decode_attn_workspace(int B, int Hq, int Hkv, int D, int k, int Tmax) {
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || k < 0 || Tmax < 0) return 256;
  return attn_partial_bytes(B, Hq, Hkv, D, k, Tmax) + ctr_bytes((size_t)B * Hkv);
}

sv_status sv_sparse_decode_attn(const void* q, int B, int Hq, const void* k_vis, const void* v_vis,
                                int64_t vis_bstride, int64_t vis_tstride, int N, int Hkv, int D,
                                const int32_t* idx, int k, const void* k_txt, const void* v_txt,
                                int64_t txt_bstride, int64_t txt_tstride, const int32_t* txt_len,
                                int Tmax, sv_dtype dtype, float scale, float* out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !out || !workspace) return fail(SV_EINVAL, "sv_sparse_decode_attn: NULL q, out or workspace");
  if (B < 1 || B > 65535 || Hq < 1 || Hkv < 1 || N < 0 || k < 0 || Tmax < 0)
    return fail(SV_EINVAL, "sv_sparse_decode_attn: bad sizes B=%d Hq=%d Hkv=%d N=%d k=%d Tmax=%d",
                B, Hq, Hkv, N, k, Tmax);
  if (k > N) return fail(SV_EINVAL, "sv_sparse_decode_attn: k=%d > N=%d", k, N);
  if (k + Tmax == 0) return fail(SV_EINVAL, "sv_sparse_decode_attn: nothing to attend (k + Tmax == 0)");
  if (k > 0 && (!k_vis || !v_vis))
    return fail(SV_EINVAL, "sv_sparse_decode_attn: NULL k_vis or v_vis");
  if (Tmax > 0 && (!k_txt || !v_txt || !txt_len))
    return fail(SV_EINVAL, "sv_sparse_decode_attn: NULL k_txt, v_txt or txt_len");
  if (Hq % Hkv) return fail(SV_EINVAL, "sv_sparse_decode_attn: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (!dtype_ok(dtype)) return fail(SV_EUNSUPPORTED, "sv_sparse_decode_attn: dtype %d", (int)dtype);
  if (D != 64 && D != 128) return fail(SV_EUNSUPPORTED, "sv_sparse_decode_attn: D=%d (64 or 128)", D);
  if (Hq / Hkv > 8) return fail(SV_EUNSUPPORTED, "sv_sparse_decode_attn: group size %d > 8", Hq / Hkv);
  const int ve = vec_elems(dtype);
  const int64_t R = (int64_t)Hkv * D;
  if (k > 0 && (vis_tstride < R || vis_bstride < 0 || vis_tstride % ve || vis_bstride % ve))
    return fail(SV_EINVAL, "sv_sparse_decode_attn: visual strides must be >= row and multiples of %d", ve);
  if (Tmax > 0 && (txt_tstride < R || txt_bstride < 0 || txt_tstride % ve || txt_bstride % ve))
    return fail(SV_EINVAL, "sv_sparse_decode_attn: text strides must be >= row and multiples of %d", ve);
  if (!aligned16(q) || (k > 0 && (!aligned16(k_vis) || !aligned16(v_vis))) ||
      (Tmax > 0 && (!aligned16(k_txt) || !aligned16(v_txt))))
    return fail(SV_EINVAL, "sv_sparse_decode_attn: q and caches must be 16-byte aligned");
  if ((k > 0 && !extent_ok(N, vis_tstride, R, dtype)) || !extent_ok(Tmax, txt_tstride, R, dtype))
    return fail(SV_EUNSUPPORTED, "sv_sparse_decode_attn: one sequence's cache slice spans 2 GiB or more");
  const size_t need = sv_sparse_decode_attn_workspace(B, Hq, Hkv, D, k, Tmax);
  if (workspace_bytes < need)
    return fail(SV_EWORKSPACE, "sv_sparse_decode_attn: workspace %zu < %zu bytes", workspace_bytes, need);
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)D);
  uint32_t* counters =
      (uint32_t*)((char*)workspace + attn_partial_bytes(B, Hq, Hkv, D, k, Tmax));
  return hip_status(sv::launch_attn(q, B, Hq, k_vis, v_vis, vis_bstride, vis_tstride, N, Hkv, D, idx,
                                    k, k_txt, v_txt, txt_bstride, txt_tstride, txt_len, Tmax,
                                    (int)dtype, sc, out, (float*)workspace, counters, 0,
                                    (hipStream_t)stream),
                    "sv_sparse_decode_attn");
}

// ---------------------------------------------------------------- dense packing
sv_status sv_pack_selected(const void* k_vis, const void* v_vis, int64_t vis_bstride,
                           int64_t vis_tstride, int N, int Hkv, int D, sv_dtype dtype,
                           const int32_t* idx, int B, int k, void* k_pack, void* v_pack,
                           void* stream) {
  if (B < 1 || N < 1 || Hkv < 1 || D < 1 || k < 0)
    return fail(SV_EINVAL, "sv_pack_selected: bad sizes B=%d N=%d Hkv=%d D=%d k=%d", B, N, Hkv, D, k);
  if (k == 0) return SV_OK;
  if (!k_vis || !v_vis || !idx || !k_pack || !v_pack)
    return fail(SV_EINVAL, "sv_pack_selected: NULL cache, idx or destination");
  if (!dtype_ok(dtype)) return fail(SV_EUNSUPPORTED, "sv_pack_selected: dtype %d", (int)dtype);
  const int ve = vec_elems(dtype);
  const int64_t R = (int64_t)Hkv * D;
  if (R % ve) return fail(SV_EINVAL, "sv_pack_selected: Hkv*D=%lld not a multiple of %d", (long long)R, ve);
  if (R > ((int64_t)1 << 24))
    return fail(SV_EUNSUPPORTED, "sv_pack_selected: row of %lld elements too long", (long long)R);
  if (vis_tstride < R || vis_bstride < 0 || vis_tstride % ve || vis_bstride % ve)
    return fail(SV_EINVAL, "sv_pack_selected: strides must be >= row and multiples of %d", ve);
  if (!aligned16(k_vis) || !aligned16(v_vis) || !aligned16(k_pack) || !aligned16(v_pack))
    return fail(SV_EINVAL, "sv_pack_selected: caches and destinations must be 16-byte aligned");
  return hip_status(sv::launch_pack(k_vis, v_vis, vis_bstride, vis_tstride, N, (int)R,
                                    dtype == SV_BF16 ? 2 : 4, idx, B, k, k_pack, v_pack,
                                    (hipStream_t)stream),
                    "sv_pack_selected");
}

// ---------------------------------------------------------------- fused layer
// Workspace of sv_retrieve_attend:
//   [status line][scores B*N][partials][control: seq B | ready B | vis_done B | comb B*Hkv]
//   [encoded index copy B*k]
//   [long-row select: control lines and histograms | candidates, chunk offsets],
// every control word on its own 128-byte line.  The score words, control
// words, index copy, and the long-row control lines and histograms are zero
// between launches (short rows: the kernel stores scores complemented and
// zeroes them once read).
static size_t fused_ctl_bytes(int B, int Hkv) { return ctr_bytes((size_t)B * (3 + Hkv)); }
static size_t fused_enc_bytes(int B, int k) { return align256((size_t)B * k * sizeof(uint32_t)); }

size_t sv_retrieve_attend_workspace(int B, int Hq, int Hkv, int D, int N, int k, int Tmax) {
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || N < 1 || k < 0 || Tmax < 0) return kStatusBytes;
  return kStatusBytes + retrieve_scores_bytes(B, N) +
         attn_partial_bytes(B, Hq, Hkv, D, k, Tmax, true, N) +
         fused_ctl_bytes(B, Hkv) + fused_enc_bytes(B, k) + sv::long_select_bytes(B, N);
}

}  // extern "C"

// The no-allocation variant resolves its workspace (the static scratch) only
// after every argument has been validated.
static sv_status scratch_workspace(size_t need, hipStream_t st, void** ws, const char* fn);

static sv_status retrieve_attend_impl(const char* fn, bool noalloc, const void* q, int B, int Hq,
                                      const void* k_vis, const void* v_vis, int64_t vis_bstride,
                                      int64_t vis_tstride, int N, int Hkv, int D, int k,
                                      const void* k_txt, const void* v_txt, int64_t txt_bstride,
                                      int64_t txt_tstride, const int32_t* txt_len, int Tmax,
                                      sv_dtype dtype, float scale, int32_t* idx_out,
                                      float* scores_out, float* out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (!q || !k_vis || !v_vis || !idx_out || !out || (!workspace && !noalloc))
    return fail(SV_EINVAL, "%s: NULL q, k_vis, v_vis, idx_out, out or workspace", fn);
  if (B < 1 || B > 65535 || Hq < 1 || Hkv < 1 || N < 1 || Tmax < 0)
    return fail(SV_EINVAL, "%s: bad sizes B=%d Hq=%d Hkv=%d N=%d Tmax=%d", fn, B, Hq, Hkv, N, Tmax);
  if (k < 1 || k > N) return fail(SV_EINVAL, "%s: k=%d outside [1, N=%d]", fn, k, N);
  if (Tmax > 0 && (!k_txt || !v_txt || !txt_len))
    return fail(SV_EINVAL, "%s: NULL k_txt, v_txt or txt_len", fn);
  if (Hq % Hkv) return fail(SV_EINVAL, "%s: Hq=%d not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (!dtype_ok(dtype)) return fail(SV_EUNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
  if (D != 64 && D != 128) return fail(SV_EUNSUPPORTED, "%s: D=%d (64 or 128)", fn, D);
  if (Hq / Hkv > 8) return fail(SV_EUNSUPPORTED, "%s: group size %d > 8", fn, Hq / Hkv);
  const int64_t R = (int64_t)Hkv * D;
  if (R > (dtype == SV_BF16 ? 8192 : 4096))
    return fail(SV_EUNSUPPORTED, "%s: row Hkv*D=%lld too long", fn, (long long)R);
  const int ve = vec_elems(dtype);
  if (vis_tstride < R || vis_bstride < 0 || vis_tstride % ve || vis_bstride % ve)
    return fail(SV_EINVAL, "%s: visual strides must be >= row and multiples of %d", fn, ve);
  if (Tmax > 0 && (txt_tstride < R || txt_bstride < 0 || txt_tstride % ve || txt_bstride % ve))
    return fail(SV_EINVAL, "%s: text strides must be >= row and multiples of %d", fn, ve);
  if (!aligned16(q) || !aligned16(k_vis) || !aligned16(v_vis) ||
      (Tmax > 0 && (!aligned16(k_txt) || !aligned16(v_txt))))
    return fail(SV_EINVAL, "%s: q and caches must be 16-byte aligned", fn);
  if (!extent_ok(N, vis_tstride, R, dtype) || !extent_ok(Tmax, txt_tstride, R, dtype))
    return fail(SV_EUNSUPPORTED, "%s: one sequence's cache slice spans 2 GiB or more", fn);
  const size_t need = sv_retrieve_attend_workspace(B, Hq, Hkv, D, N, k, Tmax);
  if (noalloc) {
    const sv_status st = scratch_workspace(need, (hipStream_t)stream, &workspace, fn);
    if (st != SV_OK) return st;
  } else if (workspace_bytes < need) {
    return fail(SV_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  }

  char* ws = (char*)workspace;
  sv::FusedLaunch f{};
  f.status = (uint32_t*)ws;
  f.spin_limit = g_wait_limit.load(std::memory_order_relaxed);
  ws += kStatusBytes;
  f.q = q;
  f.B = B;
  f.Hq = Hq;
  f.Hkv = Hkv;
  f.D = D;
  f.dtype = (int)dtype;
  f.k_vis = k_vis;
  f.v_vis = v_vis;
  f.vbs = vis_bstride;
  f.vts = vis_tstride;
  f.N = N;
  f.k = k;
  f.k_txt = k_txt;
  f.v_txt = v_txt;
  f.tbs = txt_bstride;
  f.tts = txt_tstride;
  f.txt_len = txt_len;
  f.Tmax = Tmax;
  f.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)D);
  f.idx = idx_out;
  f.scores_ws = (float*)ws;
  f.scores_out = scores_out;
  f.out = out;
  ws += retrieve_scores_bytes(B, N);
  f.part = (float*)ws;
  ws += attn_partial_bytes(B, Hq, Hkv, D, k, Tmax, true, N);
  uint32_t* ctl = (uint32_t*)ws;
  f.seq_ctr = ctl;
  f.ready = f.seq_ctr + (size_t)B * sv::kCtrStride;
  f.vis_done = f.ready + (size_t)B * sv::kCtrStride;
  f.comb_ctr = f.vis_done + (size_t)B * sv::kCtrStride;
  ws += fused_ctl_bytes(B, Hkv);
  f.idx_enc = (uint32_t*)ws;
  ws += fused_enc_bytes(B, k);
  f.long_ws = sv::long_select_bytes(B, N) ? ws : nullptr;
  return hip_status(sv::launch_fused(f, (hipStream_t)stream), fn);
}

extern "C" {

sv_status sv_retrieve_attend(const void* q, int B, int Hq, const void* k_vis, const void* v_vis,
                             int64_t vis_bstride, int64_t vis_tstride, int N, int Hkv, int D,
                             int k, const void* k_txt, const void* v_txt, int64_t txt_bstride,
                             int64_t txt_tstride, const int32_t* txt_len, int Tmax,
                             sv_dtype dtype, float scale, int32_t* idx_out, float* scores_out,
                             float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return retrieve_attend_impl("sv_retrieve_attend", false, q, B, Hq, k_vis, v_vis, vis_bstride,
                              vis_tstride, N, Hkv, D, k, k_txt, v_txt, txt_bstride, txt_tstride,
                              txt_len, Tmax, dtype, scale, idx_out, scores_out, out, workspace,
                              workspace_bytes, stream);
}

// ---------------------------------------------------------------- no-allocation variant
// For callers that cannot allocate (code under graph capture, tight serving
// loops): sv_retrieve_attend_noalloc takes its workspace from a file-scope
// device array instead of an argument.  Each device holds its own copy, at its
// own address, found once per device with hipGetSymbolAddress; every call on
// a device shares it.
sv_status sv_retrieve_attend_noalloc(const void* q, int B, int Hq, const void* k_vis,
                                     const void* v_vis, int64_t vis_bstride, int64_t vis_tstride,
                                     int N, int Hkv, int D, int k, const void* k_txt,
                                     const void* v_txt, int64_t txt_bstride, int64_t txt_tstride,
                                     const int32_t* txt_len, int Tmax, sv_dtype dtype, float scale,
                                     int32_t* idx_out, float* scores_out, float* out,
                                     void* stream) {
  return retrieve_attend_impl("sv_retrieve_attend_noalloc", true, q, B, Hq, k_vis, v_vis,
                              vis_bstride, vis_tstride, N, Hkv, D, k, k_txt, v_txt, txt_bstride,
                              txt_tstride, txt_len, Tmax, dtype, scale, idx_out, scores_out, out,
                              nullptr, 0, stream);
}

// ---------------------------------------------------------------- salience
// Workspace of sv_salience_prune: [column sums F*H*N][salience F*N][flags F*H]
// [row lse F*H*N, used by frames beyond the on-chip kernels].
size_t sv_salience_prune_workspace(int F, int H, int N) {
  if (F < 1 || H < 1 || N < 1) return 256;
  return 2 * align256((size_t)F * H * N * sizeof(float)) +
         align256((size_t)F * N * sizeof(float)) + align256((size_t)F * H * sizeof(int32_t));
}

sv_status sv_salience_prune(const void* vis_q, const void* vis_k, int F, int H, int N, int D,
                            sv_dtype dtype, float scale, int keep, float* salience_out,
                            int32_t* idx_out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!vis_q || !vis_k || !workspace) return fail(SV_EINVAL, "sv_salience_prune: NULL q, k or workspace");
  if (F < 1 || H < 1 || N < 1 || D < 1)
    return fail(SV_EINVAL, "sv_salience_prune: bad sizes F=%d H=%d N=%d D=%d", F, H, N, D);
  if ((int64_t)F * H > 2147483647LL) return fail(SV_EINVAL, "sv_salience_prune: F*H too large");
  if (keep < 0 || keep > N) return fail(SV_EINVAL, "sv_salience_prune: keep=%d outside [0, N=%d]", keep, N);
  if (keep > 0 && !idx_out) return fail(SV_EINVAL, "sv_salience_prune: NULL idx_out");
  if (dtype != SV_BF16) return fail(SV_EUNSUPPORTED, "sv_salience_prune: only SV_BF16");
  if ((int64_t)F * H * ((N + 255) / 256) > 2147483647LL)
    return fail(SV_EUNSUPPORTED, "sv_salience_prune: F*H*ceil(N/256) workgroups too many");
  if (!sv::salience_supported(N, D))
    return fail(SV_EUNSUPPORTED, "sv_salience_prune: N=%d, D=%d outside the on-chip kernel", N, D);
  if (!aligned16(vis_q) || !aligned16(vis_k))
    return fail(SV_EINVAL, "sv_salience_prune: q and k must be 16-byte aligned");
  const size_t need = sv_salience_prune_workspace(F, H, N);
  if (workspace_bytes < need)
    return fail(SV_EWORKSPACE, "sv_salience_prune: workspace %zu < %zu bytes", workspace_bytes, need);
  float* colsum = (float*)workspace;
  char* sal_ws = (char*)workspace + align256((size_t)F * H * N * sizeof(float));
  float* sal = salience_out ? salience_out : (float*)sal_ws;
  int32_t* redo = (int32_t*)(sal_ws + align256((size_t)F * N * sizeof(float)));
  float* lse = (float*)((char*)redo + align256((size_t)F * H * sizeof(int32_t)));
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)D);
  hipStream_t st = (hipStream_t)stream;
  sv_status s = hip_status(
      sv::launch_salience(vis_q, vis_k, F, H, N, D, sc, colsum, redo, lse, sal, st),
      "sv_salience_prune salience");
  if (s != SV_OK) return s;
  return hip_status(sv::launch_topk_rows(sal, F, N, N, keep, idx_out, st), "sv_salience_prune select");
}

}  // extern "C"

// ---------------------------------------------------------------- summary-token salience
// Workspace: [per-head column values F*H*N][salience F*N, when salience_out is NULL]
size_t sv_summary_salience_prune_workspace(int F, int H, int N) {
  if (F < 1 || H < 1 || N < 1) return 256;
  return align256((size_t)F * H * N * sizeof(float)) + align256((size_t)F * N * sizeof(float));
}

sv_status sv_summary_salience_prune(const void* vis_q, const void* vis_k, int F, int H, int N,
                                    int D, sv_dtype dtype, float scale, int S, int keep,
                                    float* salience_out, int32_t* idx_out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  const char* fn = "sv_summary_salience_prune";
  if (!vis_q || !vis_k || !workspace) return fail(SV_EINVAL, "%s: NULL q, k or workspace", fn);
  if (F < 1 || H < 1 || N < 1 || D < 1)
    return fail(SV_EINVAL, "%s: bad sizes F=%d H=%d N=%d D=%d", fn, F, H, N, D);
  if (S < 1 || S > N) return fail(SV_EINVAL, "%s: S=%d summary tokens outside [1, N=%d]", fn, S, N);
  if (keep < 0 || keep > N) return fail(SV_EINVAL, "%s: keep=%d outside [0, N=%d]", fn, keep, N);
  if (keep > 0 && !idx_out) return fail(SV_EINVAL, "%s: NULL idx_out", fn);
  if (!aligned16(vis_q) || !aligned16(vis_k))
    return fail(SV_EINVAL, "%s: q and k must be 16-byte aligned", fn);
  if (dtype != SV_BF16) return fail(SV_EUNSUPPORTED, "%s: dtype %d (bf16 only)", fn, (int)dtype);
  if (D % 8 || D > 128) return fail(SV_EUNSUPPORTED, "%s: D=%d (a multiple of 8, at most 128)", fn, D);
  if (S > sv::kSummaryMaxS || N > sv::kSummaryMaxN || (int64_t)S * N > sv::kSummaryMaxLogits)
    return fail(SV_EUNSUPPORTED, "%s: S=%d, N=%d outside S <= %d, N <= %d, S*N <= %d", fn, S, N,
                sv::kSummaryMaxS, sv::kSummaryMaxN, sv::kSummaryMaxLogits);
  if (F > 65535 || (int64_t)F * H > 2147483647LL)
    return fail(SV_EUNSUPPORTED, "%s: F=%d, F*H too large", fn, F);
  const size_t need = sv_summary_salience_prune_workspace(F, H, N);
  if (workspace_bytes < need)
    return fail(SV_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)D);
  float* colh = (float*)workspace;
  float* sal = salience_out
                   ? salience_out
                   : (float*)((char*)workspace + align256((size_t)F * H * N * sizeof(float)));
  return hip_status(sv::launch_summary_salience(vis_q, vis_k, F, H, N, D, S, sc, keep, colh, sal,
                                                idx_out, (hipStream_t)stream),
                    fn);
}

// ---------------------------------------------------------------- prefill attention + retrieval
// Workspace: [completion counters 2B lines][long-row select (rows of more
// than 2048 tokens)][split partials][partial retrieval scores B*NP*N]
// [scores B*N].
size_t sv_prefill_attend_retrieve_workspace(int B, int Tq, int Hq, int Hkv, int D, int N,
                                            int Tmax) {
  if (B < 1 || Tq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || N < 1 || Tmax < 0) return 256;
  const sv::PrefillPlan p = sv::prefill_plan(B, Tq, Hq, Hkv, N, Tmax);
  return align256((size_t)2 * B * sv::kCtrStride * sizeof(uint32_t)) +
         sv::prefill_long_select_bytes(B, N) +
         align256(sv::prefill_part_floats(B, Hkv, D, p) * sizeof(float)) +
         align256((size_t)B * p.NP * N * sizeof(float)) + align256((size_t)B * N * sizeof(float));
}

sv_status sv_prefill_attend_retrieve(const void* q, int B, int Tq, int Hq, const void* k_vis,
                                     const void* v_vis, int64_t vis_bstride, int64_t vis_tstride,
                                     int N, int Hkv, int D, const void* k_txt, const void* v_txt,
                                     int64_t txt_bstride, int64_t txt_tstride,
                                     const int32_t* txt_len, int Tmax, sv_dtype dtype,
                                     float scale, int k, float* out, int32_t* idx_out,
                                     float* scores_out, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  const char* fn = "sv_prefill_attend_retrieve";
  if (!q || !k_vis || !v_vis || !out || !workspace)
    return fail(SV_EINVAL, "%s: NULL q, k_vis, v_vis, out or workspace", fn);
  if (B < 1 || Tq < 1 || Hq < 1 || Hkv < 1 || N < 1 || Tmax < 0)
    return fail(SV_EINVAL, "%s: bad sizes B=%d Tq=%d Hq=%d Hkv=%d N=%d Tmax=%d", fn, B, Tq, Hq,
                Hkv, N, Tmax);
  if (k < 0 || k > N) return fail(SV_EINVAL, "%s: k=%d outside [0, N=%d]", fn, k, N);
  if (k > 0 && !idx_out) return fail(SV_EINVAL, "%s: NULL idx_out", fn);
  if (Tmax > 0 && (!k_txt || !v_txt || !txt_len))
    return fail(SV_EINVAL, "%s: NULL k_txt, v_txt or txt_len", fn);
  if (Hq % Hkv) return fail(SV_EINVAL, "%s: Hq=%d not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (dtype != SV_BF16) return fail(SV_EUNSUPPORTED, "%s: dtype %d (bf16 only)", fn, (int)dtype);
  if (D != 64 && D != 128) return fail(SV_EUNSUPPORTED, "%s: D=%d (64 or 128)", fn, D);
  const int64_t R = (int64_t)Hkv * D;
  if (vis_tstride < R || vis_bstride < 0 || vis_tstride % 8 || vis_bstride % 8)
    return fail(SV_EINVAL, "%s: visual strides must be >= row and multiples of 8", fn);
  if (Tmax > 0 && (txt_tstride < R || txt_bstride < 0 || txt_tstride % 8 || txt_bstride % 8))
    return fail(SV_EINVAL, "%s: text strides must be >= row and multiples of 8", fn);
  if (!aligned16(q) || !aligned16(k_vis) || !aligned16(v_vis) ||
      (Tmax > 0 && (!aligned16(k_txt) || !aligned16(v_txt))))
    return fail(SV_EINVAL, "%s: q and caches must be 16-byte aligned", fn);
  if ((int64_t)Tq * (Hq / Hkv) > (1 << 20))
    return fail(SV_EUNSUPPORTED, "%s: Tq * Hq / Hkv query rows per KV head above 2^20", fn);
  if (((int64_t)N + 32) * vis_tstride * 2 >= (1LL << 31) ||
      ((int64_t)Tmax + 32) * txt_tstride * 2 >= (1LL << 31))
    return fail(SV_EUNSUPPORTED, "%s: one sequence's visual or text cache spans 2 GiB or more", fn);
  const sv::PrefillPlan p = sv::prefill_plan(B, Tq, Hq, Hkv, N, Tmax);
  if ((int64_t)B * Hkv * p.RC * (p.CV + p.CT) > 2147483647LL ||
      (int64_t)B * Hkv * p.RC * p.W * 32 > 2147483647LL)
    return fail(SV_EUNSUPPORTED, "%s: too many workgroups", fn);
  const size_t need = sv_prefill_attend_retrieve_workspace(B, Tq, Hq, Hkv, D, N, Tmax);
  if (workspace_bytes < need)
    return fail(SV_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  char* ws = (char*)workspace;
  sv::PrefillArgs a{};
  a.q = (const sv::bf16_t*)q;
  a.kv = (const sv::bf16_t*)k_vis;
  a.vv = (const sv::bf16_t*)v_vis;
  a.kt = (const sv::bf16_t*)k_txt;
  a.vt = (const sv::bf16_t*)v_txt;
  a.vbs = vis_bstride;
  a.vts = vis_tstride;
  a.tbs = txt_bstride;
  a.tts = txt_tstride;
  a.txt_len = Tmax > 0 ? txt_len : nullptr;
  a.B = B;
  a.Tq = Tq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.D = D;
  a.N = N;
  a.Tmax = Tmax;
  a.c2 = (scale > 0.f ? scale : 1.0f / std::sqrt((float)D)) * 1.4426950408889634f;
  a.rows = p.rows;
  a.W = p.W;
  a.RC = p.RC;
  a.E = p.E;
  a.CV = p.CV;
  a.CT = p.CT;
  a.NP = p.NP;
  a.KW = p.KW;
  a.ctl = (uint32_t*)ws;
  ws += align256((size_t)2 * B * sv::kCtrStride * sizeof(uint32_t));
  a.long_ws = sv::prefill_long_select_bytes(B, N) ? ws : nullptr;
  ws += sv::prefill_long_select_bytes(B, N);
  a.part = (float*)ws;
  ws += align256(sv::prefill_part_floats(B, Hkv, D, p) * sizeof(float));
  a.pscore = (float*)ws;
  ws += align256((size_t)B * p.NP * N * sizeof(float));
  a.out = out;
  float* scores = scores_out ? scores_out : (float*)ws;
  a.scores = scores;
  a.k = k;
  a.idx = idx_out;
  return hip_status(sv::launch_prefill(a, scores, k, idx_out, (hipStream_t)stream), fn);
}
