// attn_api.hip -- the C ABI of libattn.so (declared in include/attn.h):
// argument validation, dtype / head-dim dispatch and kernel launch.
//
// Every check runs before any HIP call, so a rejected call enqueues nothing
// and touches no device state.  No exception crosses the ABI; nothing is
// printed; no device memory is allocated.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/attn.h"
#include "kernels.hpp"

namespace {

// MI355X (gfx950): 8 XCDs, workgroups dispatched round-robin over them.
constexpr int kXcds = 8;
// A launch's work-items must stay below 2^32; every kernel here uses 256.
constexpr uint64_t kMaxWorkgroups = (1ull << 32) / 256 - 1;

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
                        void* p, int B, int Hq, int Hkv, int N, int d, float scale, void* stream) {
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
  a.n_xcd = kXcds;
  a.stream = static_cast<hipStream_t>(stream);
  return a;
}

int to_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

int fwd_impl(bool bf16, const void* q, const void* k, const void* v, void* o, float* lse, int B,
             int Hq, int Hkv, int N, int d, float scale, void* stream) {
  int st = check_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale);
  if (st != ATTN_OK) return st;
  const bool rows64 = attn::fwd_bf16_use_rows64(d);
  const uint64_t grid = !bf16 ? attn::fwd_f32_grid(B, Hq, N)
                      : rows64 ? attn::fwd_bf16_rows64_grid(B, Hq, N)
                               : attn::fwd_bf16_rows32_grid(B, Hq, N);
  if (grid > kMaxWorkgroups) return ATTN_ERR_SHAPE;
  const int elem = bf16 ? 2 : 4;
  st = check_alias(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, N, d, elem, 0);
  if (st != ATTN_OK) return st;
  const attn::FwdArgs a = make_args(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, N, d, scale, stream);
  return to_status(!bf16 ? attn::launch_fwd_f32(a)
                   : rows64 ? attn::launch_fwd_bf16_rows64(a)
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
  const attn::FwdArgs a = make_args(q, k, v, o, lse, s, p, B, Hq, Hkv, N, d, scale, stream);
  return to_status(bf16 ? attn::launch_materialized_bf16(a) : attn::launch_materialized_f32(a));
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
    case ATTN_ERR_HIP: return "the HIP runtime reported an error at launch";
    default: return "unknown status";
  }
}

}  // extern "C"
