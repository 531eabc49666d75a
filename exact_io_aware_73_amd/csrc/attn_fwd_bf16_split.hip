// attn_fwd_bf16_split.hip -- the split-KV form of the fused forward: one key
// range of a head per workgroup, fp32 partial (O, lse) to the caller's
// workspace; attn_split_merge.hip combines the ranges.  The kernel body and
// its design notes are in rows64_pipeline.hpp.
#define ATTN_ROWS64_SPLIT 1
#include "rows64_pipeline.hpp"

namespace attn {
namespace {

template <int D, bool kNeg>
hipError_t launch_split_d(const FwdArgs& a) {
  const int n_qtiles = (int)(((uint64_t)(a.Hq / a.Hkv) * a.N + kFBr - 1) / kFBr);
  const uint64_t grid = (uint64_t)n_qtiles * a.Hkv * a.B * a.n_split;
  const float c_log2 = a.scale * 1.44269504088896341f;
  hipLaunchKernelGGL((attn_fwd_bf16_rows64_split_kernel<D, kNeg>), dim3((uint32_t)grid),
                     dim3(kFThreads), 0, a.stream, static_cast<const __bf16*>(a.q),
                     static_cast<const __bf16*>(a.k), static_cast<const __bf16*>(a.v), a.Hq,
                     a.Hkv, a.N, c_log2, n_qtiles, (uint32_t)a.n_xcd, a.n_split, a.chunk_keys,
                     (int64_t)a.B * a.Hq * a.N, a.part_o, a.part_lse);
  return hipGetLastError();
}

}  // namespace

uint64_t split_chunk_keys(int N, int n_split) {
  const int n_tiles = (N + kBc - 1) / kBc;
  const int per = (n_tiles + n_split - 1) / n_split;   // whole tiles per range
  return (uint64_t)per * kBc;
}

hipError_t launch_fwd_bf16_split(const FwdArgs& a) {
  const bool neg = a.scale < 0.0f;
  if (a.d == 128) return neg ? launch_split_d<128, true>(a) : launch_split_d<128, false>(a);
  return neg ? launch_split_d<64, true>(a) : launch_split_d<64, false>(a);
}

}  // namespace attn
