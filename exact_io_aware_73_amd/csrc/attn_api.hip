// attn_api.hip -- the C ABI of libattn.so (declared in include/attn.h):
// argument validation, dtype / head-dim dispatch and kernel launch.
//
// Every check runs before any HIP call, so a rejected call enqueues nothing
// and touches no device state.  No exception crosses the ABI; nothing is
// printed; no device memory is allocated.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/attn.h"
#include "kernels.hpp"

namespace {

// A launch's work-items must stay below 2^32; every kernel here uses 256.
constexpr uint64_t kMaxWorkgroups = (1ull << 32) / 256 - 1;

// ---------------------------------------------------------------------------
// Device facts, read once per device: the compute-unit count (the d = 128
// forward picks rows32 or rows64 by it) and the XCD count (workgroups are
// dealt round-robin over the XCDs, each with its own L2; the kernels remap
// their ids by it so that the workgroups of one K/V head share an L2).  A
// partitioned part reports its own counts.
struct DeviceFacts {
  int n_cu = 0;
  int n_xcd = 1;
  int l2_bytes = 0;   // the L2 cache of one XCD (the launch order keeps K/V there)
  hipError_t err = hipSuccess;
};
constexpr int kMaxDevices = 64;
std::once_flag g_facts_once[kMaxDevices];
DeviceFacts g_facts[kMaxDevices];

// Facts of the calling thread's current device; a HIP error otherwise.
hipError_t device_facts(DeviceFacts* out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_facts_once[dev], [dev] {
    DeviceFacts f;
    int cu = 0, xcc = 0, l2 = 0;
    f.err = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (f.err == hipSuccess)
      f.err = hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, dev);
    if (f.err == hipSuccess) f.err = hipDeviceGetAttribute(&l2, hipDeviceAttributeL2CacheSize, dev);
    if (f.err == hipSuccess && cu < 1) f.err = hipErrorInvalidDevice;
    f.n_cu = cu;
    f.n_xcd = xcc > 0 ? xcc : 1;
    f.l2_bytes = l2 > 0 ? l2 : 0;
    g_facts[dev] = f;
  });
  *out = g_facts[dev];
  return out->err;
}

}  // namespace

// ---------------------------------------------------------------------------
// The fixed scratch buffer of attn_bwd_noalloc: device memory the library
// owns, one copy per device (held until the process ends), so that entry
// point allocates nothing.  It holds the backward's per-row dot products
// D = rowsum(dO * O), 4 bytes per query row; every row is written before it
// is read, so nothing needs clearing between calls.
namespace attn {
constexpr uint64_t kScratchBytes = 16ull << 20;
__device__ __align__(256) float scratch[kScratchBytes / 4];
}  // namespace attn

namespace {

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of this device's scratch copy: looked up once per device,
// with that device current.  The host-side name of the array is a stand-in,
// not a device address, so only this pointer is ever passed to kernels.
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(attn::scratch));
    g_scratch[dev] = (g_scratch_err[dev] == hipSuccess) ? p : nullptr;
    if (g_scratch_err[dev] == hipSuccess && p == nullptr) g_scratch_err[dev] = hipErrorInvalidSymbol;
  });
  *out = g_scratch[dev];
  return g_scratch_err[dev];
}

struct Range {
  uintptr_t lo, hi;   // [lo, hi)
};

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 int B, int Hq, int Hkv, int N, int d, float scale) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

// Outputs must not overlap the inputs or each other.
int check_alias(const void* q, const void* k, const void* v, const void* o, const void* lse,
                const void* s, const void* p, int B, int Hq, int Hkv, int N, int d, int elem,
                int p_elem) {
  auto rng = [](const void* ptr, uint64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
    return Range{lo, lo + (uintptr_t)bytes};
  };
  const uint64_t qo = (uint64_t)B * Hq * N * d * elem;
  const uint64_t kv = (uint64_t)B * Hkv * N * d * elem;
  const uint64_t nn = (uint64_t)B * Hq * N * (uint64_t)N;
  Range in[3] = {rng(q, qo), rng(k, kv), rng(v, kv)};
  Range out[4];
  int n_out = 0;
  out[n_out++] = rng(o, qo);
  out[n_out++] = rng(lse, (uint64_t)B * Hq * N * 4);
  if (s) out[n_out++] = rng(s, nn * 4);
  if (p) out[n_out++] = rng(p, nn * p_elem);
  for (int i = 0; i < n_out; ++i) {
    for (const Range& r : in)
      if (overlap(out[i], r)) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(out[i], out[j])) return ATTN_ERR_ALIAS;
  }
  return ATTN_OK;
}

attn::FwdArgs make_args(const void* q, const void* k, const void* v, void* o, float* lse, float* s,
                        void* p, int B, int Hq, int Hkv, int N, int d, float scale, int n_xcd,
                        void* stream) {
  attn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.s = s;
  a.p = p;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.n_xcd = n_xcd;
  a.stream = static_cast<hipStream_t>(stream);
  return a;
}

int to_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Sizes the fused forward accepts (pointers aside).  rows32's grid (128 rows
// per workgroup) is the larger of the two bf16 kernels', so it bounds both.
int check_fwd_sizes(bool bf16, int B, int Hq, int Hkv, int N, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  const uint64_t grid = bf16 ? attn::fwd_bf16_rows32_grid(B, Hq, Hkv, N) : attn::fwd_f32_grid(B, Hq, N);
  if (grid > kMaxWorkgroups) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

int fwd_impl(bool bf16, const void* q, const void* k, const void* v, void* o, float* lse, int B,
             int Hq, int Hkv, int N, int d, float scale, void* stream) {
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale);
  if (st != ATTN_OK) return st;
  st = check_fwd_sizes(bf16, B, Hq, Hkv, N, d);
  if (st != ATTN_OK) return st;
  const int elem = bf16 ? 2 : 4;
  st = check_alias(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, N, d, elem, 0);
  if (st != ATTN_OK) return st;
  DeviceFacts f;
  if (device_facts(&f) != hipSuccess) return ATTN_ERR_HIP;
  attn::FwdArgs a =
      make_args(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, N, d, scale, f.n_xcd, stream);
  a.n_cu = f.n_cu;
  a.l2_bytes = f.l2_bytes;
  if (!bf16) return to_status(attn::launch_fwd_f32(a));
  return to_status(attn::fwd_bf16_use_rows64(B, Hq, Hkv, N, d, f.n_cu)
                       ? attn::launch_fwd_bf16_rows64(a)
                       : attn::launch_fwd_bf16_rows32(a));
}

int materialized_impl(bool bf16, const void* q, const void* k, const void* v, void* o, float* lse,
                      float* s, void* p, int B, int Hq, int Hkv, int N, int d, float scale,
                      void* stream) {
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale);
  if (st != ATTN_OK) return st;
  if (!s || !p) return ATTN_ERR_NULL;
  if (!aligned(s, 16) || !aligned(p, 16)) return ATTN_ERR_ALIGN;
  // one 256-thread workgroup per score row in the softmax kernel, and
  // ceil(N/128)^2 (bf16) or ceil(N/64)^2 (fp32) per head in the QK^T kernel
  const uint64_t rows = (uint64_t)B * Hq * N;
  const uint64_t t = bf16 ? (uint64_t)(N + 127) / 128 : (uint64_t)(N + 63) / 64;
  if (rows > kMaxWorkgroups || t * t * B * Hq > kMaxWorkgroups) return ATTN_ERR_SHAPE;
  const int elem = bf16 ? 2 : 4;
  st = check_alias(q, k, v, o, lse, s, p, B, Hq, Hkv, N, d, elem, elem);
  if (st != ATTN_OK) return st;
  DeviceFacts f;
  if (device_facts(&f) != hipSuccess) return ATTN_ERR_HIP;
  const attn::FwdArgs a = make_args(q, k, v, o, lse, s, p, B, Hq, Hkv, N, d, scale, f.n_xcd, stream);
  return to_status(bf16 ? attn::launch_materialized_bf16(a) : attn::launch_materialized_f32(a));
}

// Workspace of the split-KV path: fp32 partial O and lse per range and row.
uint64_t split_ws_bytes(int B, int Hq, int N, int d, int n_split) {
  return (uint64_t)n_split * B * Hq * (uint64_t)N * (uint64_t)(d + 1) * 4u;
}

int split_impl(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
               uint64_t ws_bytes, int n_split, int B, int Hq, int Hkv, int N, int d, float scale,
               void* stream) {
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale);
  if (st != ATTN_OK) return st;
  if (n_split < 1 || n_split > ATTN_MAX_SPLIT) return ATTN_ERR_SPLIT;
  const uint64_t chunk = attn::split_chunk_keys(N, n_split);
  const int n_eff = (int)(((uint64_t)N + chunk - 1) / chunk);   // non-empty ranges
  const uint64_t rows = (uint64_t)B * Hq * N;
  if (attn::fwd_bf16_rows64_grid(B, Hq, Hkv, N) * n_eff > kMaxWorkgroups ||
      rows * (uint64_t)(d / 8) / 256 + 1 > kMaxWorkgroups)
    return ATTN_ERR_SHAPE;
  const uint64_t need = split_ws_bytes(B, Hq, N, d, n_split);
  if (!ws || !aligned(ws, 16) || ws_bytes < need) return ATTN_ERR_WORKSPACE;
  st = check_alias(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, N, d, 2, 0);
  if (st != ATTN_OK) return st;
  {
    auto rng = [](const void* ptr, uint64_t bytes) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
      return Range{lo, lo + (uintptr_t)bytes};
    };
    const uint64_t qo = rows * d * 2, kv = (uint64_t)B * Hkv * N * d * 2;
    const Range w = rng(ws, need);
    const Range other[5] = {rng(q, qo), rng(k, kv), rng(v, kv), rng(o, qo), rng(lse, rows * 4)};
    for (const Range& r : other)
      if (overlap(w, r)) return ATTN_ERR_ALIAS;
  }
  DeviceFacts f;
  if (device_facts(&f) != hipSuccess) return ATTN_ERR_HIP;
  attn::FwdArgs a =
      make_args(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, N, d, scale, f.n_xcd, stream);
  a.n_split = n_eff;
  a.chunk_keys = (int)chunk;
  a.part_o = static_cast<float*>(ws);
  a.part_lse = static_cast<float*>(ws) + (uint64_t)n_eff * rows * d;
  st = to_status(attn::launch_fwd_bf16_split(a));
  if (st != ATTN_OK) return st;
  return to_status(attn::launch_split_merge_bf16(a));
}

// ws == nullptr with noalloc: the row dot products go to the library's
// fixed scratch buffer instead of a caller workspace.
int bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, void* ws, uint64_t ws_bytes, int B,
             int Hq, int Hkv, int N, int d, float scale, void* stream, bool noalloc = false) {
  // the forward-shaped arguments first (q, k, v, o, lse as attn_fwd checks them)
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale);
  if (st != ATTN_OK) return st;
  if (!dout || !dq || !dk || !dv) return ATTN_ERR_NULL;
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return ATTN_ERR_ALIGN;
  const uint64_t rows = (uint64_t)B * Hq * N;
  if (attn::bwd_grid(B, Hq, Hkv, N) > kMaxWorkgroups) return ATTN_ERR_SHAPE;
  const uint64_t need = rows * 4;
  if (noalloc) {
    if (need > attn::kScratchBytes) return ATTN_ERR_SCRATCH;
  } else if (!ws || !aligned(ws, 16) || ws_bytes < need) {
    return ATTN_ERR_WORKSPACE;
  }
  auto rng = [](const void* ptr, uint64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
    return Range{lo, lo + (uintptr_t)bytes};
  };
  const uint64_t qo = rows * d * 2, kv = (uint64_t)B * Hkv * N * d * 2;
  const Range in[6] = {rng(q, qo), rng(k, kv), rng(v, kv), rng(o, qo), rng(lse, rows * 4),
                       rng(dout, qo)};
  const int n_out = noalloc ? 3 : 4;   // the scratch buffer is the library's own
  const Range out[4] = {rng(dq, qo), rng(dk, kv), rng(dv, kv), rng(ws, need)};
  for (int i = 0; i < n_out; ++i) {
    for (const Range& r : in)
      if (overlap(out[i], r)) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(out[i], out[j])) return ATTN_ERR_ALIAS;
  }
  DeviceFacts f;
  if (device_facts(&f) != hipSuccess) return ATTN_ERR_HIP;
  if (noalloc && scratch_ptr(&ws) != hipSuccess) return ATTN_ERR_HIP;
  attn::FwdArgs a = make_args(q, k, v, const_cast<void*>(o), const_cast<float*>(lse), nullptr,
                              nullptr, B, Hq, Hkv, N, d, scale, f.n_xcd, stream);
  attn::BwdArgs g;
  g.dout = dout;
  g.dq = dq;
  g.dk = dk;
  g.dv = dv;
  g.dvec = static_cast<float*>(ws);
  return to_status(attn::launch_bwd_bf16(a, g));
}

int fp8_impl(const void* q8, const void* k8, const void* vt8, void* o, float* lse, float q_scale,
             float k_scale, float v_scale, int B, int Hq, int Hkv, int N, int d, float scale,
             void* stream) {
  int st = check_common(q8, k8, vt8, o, lse, B, Hq, Hkv, N, d, scale);
  if (st != ATTN_OK) return st;
  const float c = scale * q_scale * k_scale;
  if (!isfinite(q_scale) || !isfinite(k_scale) || !isfinite(v_scale) || !isfinite(c))
    return ATTN_ERR_SCALE;
  const uint64_t np = (uint64_t)attn::fp8_padded_keys(N);
  // a head's V^T (d rows of Np bytes) is addressed with 32-bit offsets
  if (np * (uint64_t)d >= (1ull << 31) || attn::fwd_fp8_grid(B, Hq, Hkv, N) > kMaxWorkgroups)
    return ATTN_ERR_SHAPE;
  auto rng = [](const void* ptr, uint64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
    return Range{lo, lo + (uintptr_t)bytes};
  };
  const uint64_t rows = (uint64_t)B * Hq * N;
  const Range in[3] = {rng(q8, rows * d), rng(k8, (uint64_t)B * Hkv * N * d),
                       rng(vt8, (uint64_t)B * Hkv * d * np)};
  const Range out[2] = {rng(o, rows * d * 2), rng(lse, rows * 4)};
  for (int i = 0; i < 2; ++i)
    for (const Range& r : in)
      if (overlap(out[i], r)) return ATTN_ERR_ALIAS;
  if (overlap(out[0], out[1])) return ATTN_ERR_ALIAS;
  DeviceFacts f;
  if (device_facts(&f) != hipSuccess) return ATTN_ERR_HIP;
  attn::FwdArgs a =
      make_args(q8, k8, vt8, o, lse, nullptr, nullptr, B, Hq, Hkv, N, d, c, f.n_xcd, stream);
  a.v_scale = v_scale;
  return to_status(attn::launch_fwd_fp8(a));
}

}  // namespace

extern "C" {

ATTN_API int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int Hq, int Hkv, int N, int d, float scale, void* stream) {
  try {
    return fwd_impl(true, q, k, v, o, lse, B, Hq, Hkv, N, d, scale, stream);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_API int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int Hq, int Hkv, int N, int d, float scale, void* stream) {
  try {
    return fwd_impl(false, q, k, v, o, lse, B, Hq, Hkv, N, d, scale, stream);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_API int attn_fwd_materialized(const void* q, const void* k, const void* v, void* o,
                                   float* lse, float* s, void* p, int B, int Hq, int Hkv, int N,
                                   int d, float scale, void* stream) {
  try {
    return materialized_impl(true, q, k, v, o, lse, s, p, B, Hq, Hkv, N, d, scale, stream);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_API int attn_fwd_materialized_f32(const float* q, const float* k, const float* v, float* o,
                                       float* lse, float* s, float* p, int B, int Hq, int Hkv,
                                       int N, int d, float scale, void* stream) {
  try {
    return materialized_impl(false, q, k, v, o, lse, s, p, B, Hq, Hkv, N, d, scale, stream);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_API int attn_fwd_fp8(const void* q8, const void* k8, const void* vt8, void* o, float* lse,
                          float q_scale, float k_scale, float v_scale, int B, int Hq, int Hkv,
                          int N, int d, float scale, void* stream) {
  try {
    return fp8_impl(q8, k8, vt8, o, lse, q_scale, k_scale, v_scale, B, Hq, Hkv, N, d, scale,
                    stream);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_API int attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                            void* workspace, unsigned long long workspace_bytes, int n_split,
                            int B, int Hq, int Hkv, int N, int d, float scale, void* stream) {
  try {
    return split_impl(q, k, v, o, lse, workspace, workspace_bytes, n_split, B, Hq, Hkv, N, d,
                      scale, stream);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_API unsigned long long attn_fwd_split_workspace_bytes(int B, int Hq, int N, int d,
                                                           int n_split) {
  if (B < 1 || Hq < 1 || N < 1 || (d != 64 && d != 128) || n_split < 1 ||
      n_split > ATTN_MAX_SPLIT)
    return 0;
  return split_ws_bytes(B, Hq, N, d, n_split);
}

ATTN_API int attn_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, unsigned long long workspace_bytes, int B, int Hq,
                      int Hkv, int N, int d, float scale, void* stream) {
  try {
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N,
                    d, scale, stream);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_API int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              int B, int Hq, int Hkv, int N, int d, float scale, void* stream) {
  try {
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, nullptr, 0, B, Hq, Hkv, N, d, scale,
                    stream, true);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_API unsigned long long attn_bwd_noalloc_max_rows(void) {
  return attn::kScratchBytes / 4;
}

ATTN_API unsigned long long attn_bwd_workspace_bytes(int B, int Hq, int N) {
  if (B < 1 || Hq < 1 || N < 1) return 0;
  return (uint64_t)B * Hq * (uint64_t)N * 4u;
}

ATTN_API int attn_device_info(int* n_cu, int* n_xcd, int* l2_bytes) {
  try {
    DeviceFacts f;
    if (device_facts(&f) != hipSuccess) return ATTN_ERR_HIP;
    if (n_cu) *n_cu = f.n_cu;
    if (n_xcd) *n_xcd = f.n_xcd;
    if (l2_bytes) *l2_bytes = f.l2_bytes;
    return ATTN_OK;
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_API int attn_fwd_plan(int B, int Hq, int Hkv, int N, int d, int* kernel) {
  try {
    if (!kernel) return ATTN_ERR_NULL;
    const int st = check_fwd_sizes(true, B, Hq, Hkv, N, d);
    if (st != ATTN_OK) return st;
    DeviceFacts f;
    if (device_facts(&f) != hipSuccess) return ATTN_ERR_HIP;
    *kernel = attn::fwd_bf16_use_rows64(B, Hq, Hkv, N, d, f.n_cu) ? ATTN_KERNEL_ROWS64
                                                                 : ATTN_KERNEL_ROWS32;
    return ATTN_OK;
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_API const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, Hq, Hkv and N must be >= 1 and the problem must fit one launch";
    case ATTN_ERR_GQA: return "Hq must be a multiple of Hkv";
    case ATTN_ERR_HEADDIM: return "head dimension d must be 64 or 128";
    case ATTN_ERR_SCALE: return "scale must be finite";
    case ATTN_ERR_ALIGN: return "q/k/v/o/s/p must be 16-byte aligned and lse 4-byte aligned";
    case ATTN_ERR_ALIAS: return "an output buffer overlaps an input or another output";
    case ATTN_ERR_HIP: return "the HIP runtime reported an error (launch or device query)";
    case ATTN_ERR_SPLIT: return "n_split must be in [1, ATTN_MAX_SPLIT]";
    case ATTN_ERR_WORKSPACE: return "workspace is NULL, not 16-byte aligned or too small";
    case ATTN_ERR_SCRATCH:
      return "the problem needs more than the library's fixed scratch buffer (B*Hq*N rows)";
    default: return "unknown status";
  }
}

}  // extern "C"
