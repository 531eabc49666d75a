// attn_split_merge.hip -- merge of the split-KV partial results.
//
// Each key range r of a row produced O_r (its weights normalised by their
// own exp-sum) and lse_r = ln(sum of its exps).  Softmax is unchanged by a
// common shift of a row's scores, so the full row is the weighted average
//   lse = ln(sum_r e^{lse_r}),   O = sum_r e^{lse_r - lse} O_r
// (the rescale rule of the online softmax, applied once per range: blog
// "attention 的显存线性化", section 三 and its recurrences).
//
// One thread per (row, 8 consecutive d): it reads the row's n_split lse
// values and its 8-column slice of every O_r, and writes 16 bytes of bf16 O
// (and the lse, from the row's first thread).  Bound by HBM: the partials
// are read once.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads)
void attn_split_merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                             __bf16* __restrict__ o, float* __restrict__ lse, int64_t n_rows,
                             int n_split) {
  constexpr int kPer = D / 8;   // threads per row
  const int64_t t = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  const int64_t row = t / kPer;
  if (row >= n_rows) return;
  const int c0 = (int)(t % kPer) * 8;

  // log2 domain: l2 = lse * log2(e)
  constexpr float kLog2e = 1.44269504088896341f;
  float mx = -INFINITY;
  for (int r = 0; r < n_split; ++r) mx = fmaxf(mx, part_lse[(int64_t)r * n_rows + row] * kLog2e);
  float sum = 0.0f;
  for (int r = 0; r < n_split; ++r) sum += exp2_fast(part_lse[(int64_t)r * n_rows + row] * kLog2e - mx);
  const float l2 = mx + log2_fast(sum);

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < n_split; ++r) {
    const float wgt = exp2_fast(part_lse[(int64_t)r * n_rows + row] * kLog2e - l2);
    const float* src = part_o + ((int64_t)r * n_rows + row) * D + c0;
    acc0 += wgt * *reinterpret_cast<const f32x4*>(src);
    acc1 += wgt * *reinterpret_cast<const f32x4*>(src + 4);
  }
  u32x4 pk;
  pk[0] = pack_bf16x2(acc0[0], acc0[1]);
  pk[1] = pack_bf16x2(acc0[2], acc0[3]);
  pk[2] = pack_bf16x2(acc1[0], acc1[1]);
  pk[3] = pack_bf16x2(acc1[2], acc1[3]);
  *reinterpret_cast<u32x4*>(o + row * D + c0) = pk;
  if (c0 == 0) lse[row] = l2 * 0.69314718055994531f;
}

template <int D>
hipError_t launch_d(const FwdArgs& a) {
  const int64_t n_rows = (int64_t)a.B * a.Hq * a.N;
  const uint64_t threads = (uint64_t)n_rows * (D / 8);
  const uint64_t grid = (threads + kMergeThreads - 1) / kMergeThreads;
  hipLaunchKernelGGL((attn_split_merge_kernel<D>), dim3((uint32_t)grid), dim3(kMergeThreads), 0,
                     a.stream, a.part_o, a.part_lse, static_cast<__bf16*>(a.o), a.lse, n_rows,
                     a.n_split);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split_merge_bf16(const FwdArgs& a) {
  return a.d == 128 ? launch_d<128>(a) : launch_d<64>(a);
}

}  // namespace attn
