// attn_fwd_bf16_rows64.hip -- the attn_fwd kernel for head dim 128 on long
// keys with a grid that fills the GPU: every key of a head per workgroup.
// The kernel body and its design notes are in rows64_pipeline.hpp (whose
// d = 64 form serves only the split-KV path).
#define ATTN_ROWS64_SPLIT 0
#include "rows64_pipeline.hpp"

namespace attn {
namespace {

template <int D, bool kNeg>
hipError_t launch_d(const FwdArgs& a) {
  const int n_qtiles = (int)(((uint64_t)(a.Hq / a.Hkv) * a.N + kFBr - 1) / kFBr);
  const uint64_t grid = (uint64_t)n_qtiles * a.Hkv * a.B;
  const float c_log2 = a.scale * 1.44269504088896341f;
  // reverse every other round where a K/V head fits one XCD's L2 and there is
  // no partial last tile
  const uint64_t kv_bytes = 2ull * a.N * D * 2;
  const bool rev = a.N % kBc == 0 && a.N > kBc && a.l2_bytes > 0 &&
                   kv_bytes <= (uint64_t)a.l2_bytes && a.n_cu >= a.n_xcd;
  const uint32_t rev_every = rev ? (uint32_t)(a.n_cu / a.n_xcd) : 0u;
  hipLaunchKernelGGL((attn_fwd_bf16_rows64_kernel<D, kNeg>), dim3((uint32_t)grid), dim3(kFThreads), 0,
                     a.stream, static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<__bf16*>(a.o), a.lse, a.Hq,
                     a.Hkv, a.N, c_log2, n_qtiles, (uint32_t)a.n_xcd, rev_every);
  return hipGetLastError();
}

}  // namespace

uint64_t fwd_bf16_rows64_grid(int B, int Hq, int Hkv, int N) {
  return ((uint64_t)(Hq / Hkv) * N + kFBr - 1) / kFBr * Hkv * B;
}

hipError_t launch_fwd_bf16_rows64(const FwdArgs& a) {
  if (a.d != 128) return hipErrorInvalidValue;   // head dim 64 runs rows32
  const bool neg = a.scale < 0.0f;
  return neg ? launch_d<128, true>(a) : launch_d<128, false>(a);
}

}  // namespace attn
