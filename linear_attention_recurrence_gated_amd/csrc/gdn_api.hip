// C ABI of libgdn (declared in include/gdn.h): host-side validation, then kernel launches
// on the caller's stream.  Validation happens before any HIP call, so a rejected call
// touches neither memory nor the device.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "gdn.h"
#include "gdn_kernels.h"

namespace gdn {

// Compute units per device, filled on first use (0 = not yet queried).  Racing first calls
// store the same value, so relaxed atomics suffice.
constexpr int kMaxDevices = 64;
static std::atomic<int> g_cu_count[kMaxDevices];

hipError_t device_cu_count(hipStream_t stream, int* cus) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *cus = cached;
      return hipSuccess;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n < 1) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return hipSuccess;
}

// Workspace of gdn_layer_chunked_noalloc: a file-scope device array, one copy per device,
// held from the first call on that device until the process ends.  It holds the chunked
// kernels' operators for up to kStaticMaxVHeads value heads (both halves of the
// double-buffered super-block workspace: 2 x 64 chunks x 64 heads x 8704 bytes = 68 MiB).
// In host code `scratch` names a host-side stand-in, never device memory: every use goes
// through the address hipGetSymbolAddress returns for the device.
constexpr int kStaticMaxVHeads = 64;
constexpr size_t kStaticScratchBytes =
    2 * (size_t)kChunksPerSB * kStaticMaxVHeads * kSlot * sizeof(float);
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

static std::mutex g_scratch_mu;
static std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the device that `stream` runs on, resolved once per
// device with that device current.
hipError_t static_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (void* p = g_scratch_ptr[dev].load(std::memory_order_acquire)) {
    *out = p;
    return hipSuccess;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (void* p = g_scratch_ptr[dev].load(std::memory_order_acquire)) {
    *out = p;
    return hipSuccess;
  }
  int cur = 0;
  if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != dev) {
    const hipError_t e2 = hipSetDevice(cur);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  *out = p;
  return hipSuccess;
}

}  // namespace gdn

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return GDN_ERR_HIP;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlap(Range a, Range b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(int64_t T, int n_k_heads, int n_v_heads, int dk, int dv) {
  if (T < 0 || n_k_heads < 1 || n_v_heads < 1) return GDN_ERR_BAD_SHAPE;
  if (dk != gdn::kDim || dv != gdn::kDim) return GDN_ERR_BAD_SHAPE;
  if (n_v_heads % n_k_heads != 0) return GDN_ERR_BAD_SHAPE;
  if (n_v_heads / n_k_heads > gdn::kMaxGroup) return GDN_ERR_BAD_SHAPE;
  // 32-bit element offsets over a whole call ...
  if (T * (int64_t)n_v_heads * dv >= ((int64_t)1 << 31)) return GDN_ERR_BAD_SHAPE;
  // ... and 32-bit byte counts over one super-block (the chunked kernels' buffer ranges of
  // the o, v and y rows of a 2048-token super-block; n_k_heads <= n_v_heads)
  if ((int64_t)gdn::kSuperBlock * n_v_heads * dv * (int64_t)sizeof(float) >= ((int64_t)1 << 31))
    return GDN_ERR_BAD_SHAPE;
  return GDN_OK;
}

// Shared validation of the two recurrence entry points.
int check_recurrence(const float* q, const float* k, const float* v, const float* g,
                     const float* beta, const float* state_in, const float* state_out,
                     const float* o, int64_t T, int n_k_heads, int n_v_heads, int dk, int dv,
                     const void* workspace, size_t ws_bytes, bool chunked) {
  if (int s = check_shape(T, n_k_heads, n_v_heads, dk, dv)) return s;
  if (!state_in || !state_out) return GDN_ERR_NULL_POINTER;
  if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL_POINTER;
  if (chunked && T > 0 && !workspace) return GDN_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, g, beta, state_in, state_out, o, chunked ? workspace : nullptr};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_MISALIGNED;
  if (chunked && T > 0 &&
      ws_bytes < gdn_chunked_workspace_bytes(n_k_heads, n_v_heads, dk, dv))
    return GDN_ERR_WORKSPACE;

  const size_t f = sizeof(float);
  const size_t qk_b = (size_t)T * n_k_heads * dk * f, v_b = (size_t)T * n_v_heads * dv * f;
  const size_t gb_b = (size_t)T * n_v_heads * f, s_b = (size_t)n_v_heads * dk * dv * f;
  const Range in[] = {range_of(q, q ? qk_b : 0), range_of(k, k ? qk_b : 0),
                      range_of(v, v ? v_b : 0),  range_of(g, g ? gb_b : 0),
                      range_of(beta, beta ? gb_b : 0), range_of(state_in, s_b)};
  const Range r_o = range_of(o, o ? v_b : 0), r_s = range_of(state_out, s_b);
  for (const Range& r : in)
    if (overlap(r_o, r)) return GDN_ERR_ALIASING;
  for (int i = 0; i < 5; ++i)  // q, k, v, g, beta
    if (overlap(r_s, in[i])) return GDN_ERR_ALIASING;
  // state_out may be state_in itself (in place) but must not partly overlap it
  if (state_out != state_in && overlap(r_s, in[5])) return GDN_ERR_ALIASING;
  if (overlap(r_o, r_s)) return GDN_ERR_ALIASING;
  if (chunked && T > 0) {
    const Range r_w = range_of(workspace, ws_bytes);
    for (const Range& r : in)
      if (overlap(r_w, r)) return GDN_ERR_ALIASING;
    if (overlap(r_w, r_o) || overlap(r_w, r_s)) return GDN_ERR_ALIASING;
  }
  return GDN_OK;
}

// The norm operands of gdn_layer_chunked (after check_recurrence has passed): z and w are
// read, y is written; y must overlap nothing else, and the recurrence's writes (o, the
// state, the workspace) must not overlap z or w.
int check_layer_norm(const float* q, const float* k, const float* v, const float* g,
                     const float* beta, const float* state_in, const float* state_out,
                     const float* o, const void* workspace, size_t ws_bytes, const float* z,
                     const float* w, float eps, const uint16_t* y, int64_t T, int n_k_heads,
                     int n_v_heads) {
  if (!(eps >= 0.0f) || !isfinite(eps)) return GDN_ERR_BAD_SHAPE;
  if (!w || !y || (T > 0 && !z)) return GDN_ERR_NULL_POINTER;
  const void* ptrs[] = {z, w, y};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_MISALIGNED;
  if (T == 0) return GDN_OK;
  const size_t f = sizeof(float), dk = gdn::kDim, dv = gdn::kDim;
  const size_t qk_b = (size_t)T * n_k_heads * dk * f, v_b = (size_t)T * n_v_heads * dv * f;
  const size_t gb_b = (size_t)T * n_v_heads * f, s_b = (size_t)n_v_heads * dk * dv * f;
  const Range r_y = range_of(y, (size_t)T * n_v_heads * dv * sizeof(uint16_t));
  const Range r_z = range_of(z, v_b), r_w = range_of(w, (size_t)n_v_heads * dv * f);
  const Range others[] = {range_of(q, qk_b),      range_of(k, qk_b),
                          range_of(v, v_b),       range_of(g, gb_b),
                          range_of(beta, gb_b),   range_of(state_in, s_b),
                          range_of(state_out, s_b), range_of(o, v_b),
                          range_of(workspace, ws_bytes), r_z, r_w};
  for (const Range& r : others)
    if (overlap(r_y, r)) return GDN_ERR_ALIASING;
  const Range writes[] = {range_of(state_out, s_b), range_of(o, v_b),
                          range_of(workspace, ws_bytes)};
  for (const Range& r : writes)
    if (overlap(r, r_z) || overlap(r, r_w)) return GDN_ERR_ALIASING;
  return GDN_OK;
}

int copy_state_if_needed(const float* state_in, float* state_out, int n_v_heads, int dk,
                         int dv, hipStream_t s) {
  if (state_out == state_in) return GDN_OK;
  const hipError_t e = hipMemcpyAsync(state_out, state_in,
                                      (size_t)n_v_heads * dk * dv * sizeof(float),
                                      hipMemcpyDeviceToDevice, s);
  return e == hipSuccess ? GDN_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int gdn_recurrence_seq(const float* q, const float* k, const float* v, const float* g,
                       const float* beta, const float* state_in, float* state_out, float* o,
                       int64_t T, int n_k_heads, int n_v_heads, int dk, int dv, void* stream) {
  if (int st = check_recurrence(q, k, v, g, beta, state_in, state_out, o, T, n_k_heads,
                                n_v_heads, dk, dv, nullptr, 0, false))
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) return copy_state_if_needed(state_in, state_out, n_v_heads, dk, dv, s);
  gdn::SeqArgs a{q, k, v, g, beta, state_in, state_out, o, (int)T, n_k_heads};
  const hipError_t e = gdn::launch_seq(a, n_v_heads / n_k_heads, s);
  return e == hipSuccess ? GDN_OK : hip_fail(e);
}

size_t gdn_chunked_workspace_bytes(int n_k_heads, int n_v_heads, int dk, int dv) {
  if (check_shape(0, n_k_heads, n_v_heads, dk, dv) != GDN_OK) return 0;
  // two halves: one super-block's operators are scanned while the next one's are formed
  return 2 * (size_t)gdn::kChunksPerSB * n_v_heads * gdn::kSlot * sizeof(float);
}

}  // extern "C"

namespace {

// The norm half of gdn_layer_chunked (NULL y: the recurrence alone).
struct NormOut {
  const float* z;
  const float* w;
  float eps;
  uint16_t* y;
};

int chunked_impl(const float* q, const float* k, const float* v, const float* g,
                 const float* beta, const float* state_in, float* state_out, float* o,
                 int64_t T, int n_k_heads, int n_v_heads, int dk, int dv, void* workspace,
                 size_t workspace_bytes, const NormOut& nrm, void* const* scan_events,
                 int n_scan_events, void* stream) {
  if (int st = check_recurrence(q, k, v, g, beta, state_in, state_out, o, T, n_k_heads,
                                n_v_heads, dk, dv, workspace, workspace_bytes, true))
    return st;
  if (nrm.y || nrm.z || nrm.w) {
    if (int st = check_layer_norm(q, k, v, g, beta, state_in, state_out, o, workspace,
                                  workspace_bytes, nrm.z, nrm.w, nrm.eps, nrm.y, T, n_k_heads,
                                  n_v_heads))
      return st;
  }
  if (n_scan_events > 0 && !scan_events) return GDN_ERR_NULL_POINTER;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) return copy_state_if_needed(state_in, state_out, n_v_heads, dk, dv, s);
  // Workspace halves alternate between super-blocks: launch sb scans super-block sb from
  // half sb % 2 while its extra workgroups prepare super-block sb + 1 into the other half.
  const size_t half_floats = (size_t)gdn::kChunksPerSB * n_v_heads * gdn::kSlot;
  const int nsb = (int)((T + gdn::kSuperBlock - 1) / gdn::kSuperBlock);
  auto sb_args = [&](int sb) {
    const int64_t t0 = (int64_t)sb * gdn::kSuperBlock;
    const int n = (int)((T - t0) < gdn::kSuperBlock ? (T - t0) : gdn::kSuperBlock);
    return gdn::ChunkArgs{q, k, v, g, beta, t0 == 0 ? state_in : state_out, state_out, o,
                          static_cast<float*>(workspace) + (sb & 1) * half_floats, (int)t0, n,
                          n_k_heads, n_v_heads};
  };
  // The norm of super-block sb - 1 runs inside launch sb (its o is complete by then); the
  // last super-block's norm is a launch of its own.
  auto norm_rows = [&](int sb) {
    const int64_t t0 = (int64_t)sb * gdn::kSuperBlock;
    const int n = (int)((T - t0) < gdn::kSuperBlock ? (T - t0) : gdn::kSuperBlock);
    const size_t off = (size_t)t0 * n_v_heads * dv;
    return gdn::NormArgs{o + off, nrm.z + off, nrm.w, nrm.y + off, nrm.eps, n * n_v_heads,
                         n_v_heads};
  };
  const gdn::ChunkArgs first = sb_args(0);
  hipError_t e = gdn::launch_chunk_prep(first, s);
  if (e != hipSuccess) return hip_fail(e);
  for (int sb = 0; sb < nsb; ++sb) {
    const gdn::ChunkArgs a = sb_args(sb);
    const gdn::ChunkArgs next = sb + 1 < nsb ? sb_args(sb + 1) : a;
    const gdn::NormArgs prev = nrm.y && sb > 0 ? norm_rows(sb - 1) : gdn::NormArgs{};
    const bool timed = 2 * sb + 1 < n_scan_events;
    if (timed && (e = hipEventRecord(static_cast<hipEvent_t>(scan_events[2 * sb]), s)) !=
                     hipSuccess)
      return hip_fail(e);
    e = gdn::launch_chunk_scan_fused(a, sb + 1 < nsb ? &next : nullptr,
                                     nrm.y && sb > 0 ? &prev : nullptr, s);
    if (e != hipSuccess) return hip_fail(e);
    if (timed && (e = hipEventRecord(static_cast<hipEvent_t>(scan_events[2 * sb + 1]), s)) !=
                     hipSuccess)
      return hip_fail(e);
  }
  if (nrm.y) {
    const gdn::NormArgs last = norm_rows(nsb - 1);
    if ((e = gdn::launch_out_norm(last, s)) != hipSuccess) return hip_fail(e);
  }
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_recurrence_chunked(const float* q, const float* k, const float* v, const float* g,
                           const float* beta, const float* state_in, float* state_out,
                           float* o, int64_t T, int n_k_heads, int n_v_heads, int dk, int dv,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return chunked_impl(q, k, v, g, beta, state_in, state_out, o, T, n_k_heads, n_v_heads, dk,
                      dv, workspace, workspace_bytes, NormOut{}, nullptr, 0, stream);
}

int gdn_recurrence_chunked_timed(const float* q, const float* k, const float* v,
                                 const float* g, const float* beta, const float* state_in,
                                 float* state_out, float* o, int64_t T, int n_k_heads,
                                 int n_v_heads, int dk, int dv, void* workspace,
                                 size_t workspace_bytes, void* const* scan_events,
                                 int n_scan_events, void* stream) {
  return chunked_impl(q, k, v, g, beta, state_in, state_out, o, T, n_k_heads, n_v_heads, dk,
                      dv, workspace, workspace_bytes, NormOut{}, scan_events, n_scan_events,
                      stream);
}

int gdn_recurrence(const float* q, const float* k, const float* v, const float* g,
                   const float* beta, const float* state_in, float* state_out, float* o,
                   int64_t T, int n_k_heads, int n_v_heads, int dk, int dv, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (T < GDN_CHUNKED_MIN_T)
    return gdn_recurrence_seq(q, k, v, g, beta, state_in, state_out, o, T, n_k_heads,
                              n_v_heads, dk, dv, stream);
  return gdn_recurrence_chunked(q, k, v, g, beta, state_in, state_out, o, T, n_k_heads,
                                n_v_heads, dk, dv, workspace, workspace_bytes, stream);
}

int gdn_layer_chunked(const float* q, const float* k, const float* v, const float* g,
                      const float* beta, const float* state_in, float* state_out, float* o,
                      const float* z, const float* w, float eps, uint16_t* y, int64_t T,
                      int n_k_heads, int n_v_heads, int dk, int dv, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!y || !w || (T > 0 && !z)) return GDN_ERR_NULL_POINTER;
  return chunked_impl(q, k, v, g, beta, state_in, state_out, o, T, n_k_heads, n_v_heads, dk,
                      dv, workspace, workspace_bytes, NormOut{z, w, eps, y}, nullptr, 0,
                      stream);
}

int gdn_layer_chunked_timed(const float* q, const float* k, const float* v, const float* g,
                            const float* beta, const float* state_in, float* state_out,
                            float* o, const float* z, const float* w, float eps, uint16_t* y,
                            int64_t T, int n_k_heads, int n_v_heads, int dk, int dv,
                            void* workspace, size_t workspace_bytes,
                            void* const* scan_events, int n_scan_events, void* stream) {
  if (!y || !w || (T > 0 && !z)) return GDN_ERR_NULL_POINTER;
  return chunked_impl(q, k, v, g, beta, state_in, state_out, o, T, n_k_heads, n_v_heads, dk,
                      dv, workspace, workspace_bytes, NormOut{z, w, eps, y}, scan_events,
                      n_scan_events, stream);
}

int gdn_layer_chunked_noalloc(const float* q, const float* k, const float* v, const float* g,
                              const float* beta, const float* state_in, float* state_out,
                              float* o, const float* z, const float* w, float eps, uint16_t* y,
                              int64_t T, int n_k_heads, int n_v_heads, int dk, int dv,
                              void* stream) {
  // Every argument is validated before the first HIP call (the workspace is the library's
  // own array, so it takes part in no caller-side check).
  if (int st = check_shape(T, n_k_heads, n_v_heads, dk, dv)) return st;
  if (n_v_heads > gdn::kStaticMaxVHeads) return GDN_ERR_WORKSPACE;
  if (!y || !w || (T > 0 && !z)) return GDN_ERR_NULL_POINTER;
  if (int st = check_recurrence(q, k, v, g, beta, state_in, state_out, o, T, n_k_heads,
                                n_v_heads, dk, dv, nullptr, 0, false))
    return st;
  if (int st = check_layer_norm(q, k, v, g, beta, state_in, state_out, o, nullptr, 0, z, w, eps,
                                y, T, n_k_heads, n_v_heads))
    return st;
  void* ws = nullptr;
  if (const hipError_t e = gdn::static_scratch(static_cast<hipStream_t>(stream), &ws))
    return hip_fail(e);
  return chunked_impl(q, k, v, g, beta, state_in, state_out, o, T, n_k_heads, n_v_heads, dk,
                      dv, ws, gdn::kStaticScratchBytes, NormOut{z, w, eps, y}, nullptr, 0,
                      stream);
}

int gdn_out_norm(const float* o, const float* z, const float* w, float eps, uint16_t* y,
                 int64_t T, int n_v_heads, int dv, void* stream) {
  if (T < 0 || n_v_heads < 1 || dv != gdn::kDim) return GDN_ERR_BAD_SHAPE;
  if (!(eps >= 0.0f) || !isfinite(eps)) return GDN_ERR_BAD_SHAPE;
  if (T * (int64_t)n_v_heads * dv >= ((int64_t)1 << 31)) return GDN_ERR_BAD_SHAPE;
  if (!w) return GDN_ERR_NULL_POINTER;
  if (T > 0 && (!o || !z || !y)) return GDN_ERR_NULL_POINTER;
  const void* ptrs[] = {o, z, w, y};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_MISALIGNED;
  if (T == 0) return GDN_OK;
  const size_t n = (size_t)T * n_v_heads * dv;
  const Range r_y = range_of(y, n * sizeof(uint16_t));
  if (overlap(r_y, range_of(o, n * sizeof(float))) ||
      overlap(r_y, range_of(z, n * sizeof(float))) ||
      overlap(r_y, range_of(w, (size_t)n_v_heads * dv * sizeof(float))))
    return GDN_ERR_ALIASING;
  gdn::NormArgs a{o, z, w, y, eps, (int)(T * n_v_heads), n_v_heads};
  const hipError_t e = gdn::launch_out_norm(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : hip_fail(e);
}

int gdn_pre(const float* x, const float* conv_w, const float* hist_in, float* hist_out,
            const float* a, const float* b, const float* A_log, const float* dt_bias,
            int activation, float eps, float* q, float* k, float* v, float* g, float* beta,
            int64_t T, int n_k_heads, int n_v_heads, int dk, int dv, void* stream) {
  if (T < 0 || T >= ((int64_t)1 << 31) || n_k_heads < 1 || n_v_heads < 1)
    return GDN_ERR_BAD_SHAPE;
  if (dk != gdn::kDim || dv != gdn::kDim) return GDN_ERR_BAD_SHAPE;
  if (n_k_heads > 65536 || n_v_heads > 65536) return GDN_ERR_BAD_SHAPE;
  if (activation != 0 && activation != 1) return GDN_ERR_BAD_SHAPE;
  if (!(eps >= 0.0f) || !isfinite(eps)) return GDN_ERR_BAD_SHAPE;
  // the kernel indexes its waves and workgroups with 32-bit integers (gate workgroups
  // counted as if the gates were given)
  int conv_blocks = 0, blocks = 0;
  if (!gdn::pre_grid(T, n_k_heads, n_v_heads, true, &conv_blocks, &blocks))
    return GDN_ERR_BAD_SHAPE;
  const size_t f = sizeof(float);
  const size_t C = (size_t)(2 * n_k_heads + n_v_heads) * gdn::kDim;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {  // only the history: every other pointer may be NULL (empty tensors)
    if (!hist_in || !hist_out) return GDN_ERR_NULL_POINTER;
    if (!aligned16(hist_in) || !aligned16(hist_out)) return GDN_ERR_MISALIGNED;
    if (overlap(range_of(hist_in, 3 * C * f), range_of(hist_out, 3 * C * f)))
      return GDN_ERR_ALIASING;
    const hipError_t e = hipMemcpyAsync(hist_out, hist_in, 3 * C * f, hipMemcpyDeviceToDevice, s);
    return e == hipSuccess ? GDN_OK : hip_fail(e);
  }
  const bool gates = a || b || A_log || dt_bias || g || beta;
  if (gates && !(a && b && A_log && dt_bias && g && beta)) return GDN_ERR_NULL_POINTER;
  if (!x || !conv_w || !hist_in || !hist_out || !q || !k || !v) return GDN_ERR_NULL_POINTER;
  const void* ptrs[] = {x, conv_w, hist_in, hist_out, a, b, A_log, dt_bias, q, k, v, g, beta};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_ERR_MISALIGNED;
  const size_t qk_b = (size_t)T * n_k_heads * gdn::kDim * f;
  const size_t v_b = (size_t)T * n_v_heads * gdn::kDim * f, gb_b = (size_t)T * n_v_heads * f;
  const Range in[] = {range_of(x, (size_t)T * C * f), range_of(conv_w, C * 4 * f),
                      range_of(hist_in, 3 * C * f), range_of(a, a ? gb_b : 0),
                      range_of(b, b ? gb_b : 0), range_of(A_log, A_log ? n_v_heads * f : 0),
                      range_of(dt_bias, dt_bias ? n_v_heads * f : 0)};
  const Range out[] = {range_of(hist_out, 3 * C * f), range_of(q, q ? qk_b : 0),
                       range_of(k, k ? qk_b : 0), range_of(v, v ? v_b : 0),
                       range_of(g, g ? gb_b : 0), range_of(beta, beta ? gb_b : 0)};
  for (size_t i = 0; i < sizeof(out) / sizeof(out[0]); ++i) {
    for (const Range& r : in)
      if (overlap(out[i], r)) return GDN_ERR_ALIASING;
    for (size_t j = i + 1; j < sizeof(out) / sizeof(out[0]); ++j)
      if (overlap(out[i], out[j])) return GDN_ERR_ALIASING;
  }
  gdn::PreArgs pa{x, conv_w, hist_in, hist_out, gates ? a : nullptr, b, A_log, dt_bias,
                  q, k, v, g, beta, activation, eps, (int)T, n_k_heads, n_v_heads};
  const hipError_t e = gdn::launch_pre(pa, s);
  return e == hipSuccess ? GDN_OK : hip_fail(e);
}

const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL_POINTER: return "a required pointer is NULL";
    case GDN_ERR_BAD_SHAPE: return "unsupported shape or argument value";
    case GDN_ERR_MISALIGNED: return "a pointer is not 16-byte aligned";
    case GDN_ERR_ALIASING: return "an output overlaps an input or another output";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    default: return "unknown status";
  }
}

int gdn_last_hip_error(void) { return g_last_hip_error; }

int gdn_abi_version(void) { return 1; }

}  // extern "C"
