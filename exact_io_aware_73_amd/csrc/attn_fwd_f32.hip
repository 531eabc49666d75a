// attn_fwd_f32.hip -- fused, tiled attention forward with float32 I/O and
// float32 arithmetic throughout (vector FMA, no reduced-precision products).
//
// Same IO-aware schedule as the bf16 kernel (blog "attention 的显存线性化",
// section 三): a workgroup owns 64 query rows of one head and streams all
// key/value tiles of the head through LDS with a running max m and exp-sum
// l per row; S and P never leave registers.
//
// Work split: four lanes (a quad) share one query row; lane r of the quad
// holds dims {16 i + 4 r .. 16 i + 4 r + 3} of q and of the O accumulator, so
// the quad's four 16-byte LDS reads of a K / V row are contiguous and every
// quad of the wave reads the same row (an LDS broadcast).  A score is the
// quad's four partial dot products summed with two lane exchanges.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kF32Threads = 256;
constexpr int kF32Rows = kF32Threads / 4;   // query rows per workgroup
constexpr int kF32Bc = 32;                  // keys per tile

template <int D>
__global__ __launch_bounds__(kF32Threads)
void attn_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                         const float* __restrict__ v, float* __restrict__ o,
                         float* __restrict__ lse, int Hq, int Hkv, int N, float c_log2,
                         int n_qtiles, uint32_t n_xcd) {
  constexpr int kPer = D / 16;            // float4 groups per lane
  __shared__ __align__(16) float ks[kF32Bc * D];
  __shared__ __align__(16) float vs[kF32Bc * D];

  const int tid = threadIdx.x;
  const int quad_lane = tid & 3;
  const int row_in_wg = tid >> 2;

  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x, n_xcd);
  // the query heads that share a K/V head are numbered fastest, then query
  // tiles: workgroups that stream the same K/V rows at the same time run
  // side by side on one XCD and share its L2
  const int group = Hq / Hkv;
  const int hg = (int)(logical % (uint32_t)group);
  uint32_t rest = logical / (uint32_t)group;
  const int qt = (int)(rest % (uint32_t)n_qtiles);
  rest /= (uint32_t)n_qtiles;
  const int kvh = (int)(rest % (uint32_t)Hkv);
  const int b = (int)(rest / (uint32_t)Hkv);
  const int h = kvh * group + hg;

  const int64_t head_q = ((int64_t)b * Hq + h) * (int64_t)N;
  const int64_t head_kv = ((int64_t)b * Hkv + kvh) * (int64_t)N;
  const float* kh = k + head_kv * D;
  const float* vh = v + head_kv * D;

  const int qrow = qt * kF32Rows + row_in_wg;
  const bool qvalid = qrow < N;

  f32x4 qv[kPer], acc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    qv[i] = qvalid ? *reinterpret_cast<const f32x4*>(q + (head_q + qrow) * D + 16 * i + 4 * quad_lane)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m_run = -INFINITY;   // running max of the log2-scaled scores
  float l_run = 0.0f;

  const int n_tiles = (N + kF32Bc - 1) / kF32Bc;
  for (int jt = 0; jt < n_tiles; ++jt) {
    const int j0 = jt * kF32Bc;
    // stage K and V rows j0 .. j0 + kF32Bc - 1 (zeros past N)
    for (int c = tid; c < kF32Bc * D / 4; c += kF32Threads) {
      const int row = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
      const bool ok = j0 + row < N;
      const int64_t off = (int64_t)(j0 + row) * D + col;
      *reinterpret_cast<f32x4*>(ks + row * D + col) =
          ok ? *reinterpret_cast<const f32x4*>(kh + off) : f32x4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(vs + row * D + col) =
          ok ? *reinterpret_cast<const f32x4*>(vh + off) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();

    float s[kF32Bc];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32Bc; ++j) {
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const f32x4 kk = *reinterpret_cast<const f32x4*>(ks + j * D + 16 * i + 4 * quad_lane);
        part = __builtin_fmaf(qv[i][0], kk[0], part);
        part = __builtin_fmaf(qv[i][1], kk[1], part);
        part = __builtin_fmaf(qv[i][2], kk[2], part);
        part = __builtin_fmaf(qv[i][3], kk[3], part);
      }
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      s[j] = (j0 + j < N) ? part * c_log2 : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2_fast(m_run - m_new);   // 0 on the first tile
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < kF32Bc; ++j) {
      const float p = exp2_fast(s[j] - m_run);
      l_run += p;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const f32x4 vv = *reinterpret_cast<const f32x4*>(vs + j * D + 16 * i + 4 * quad_lane);
        acc[i][0] = __builtin_fmaf(p, vv[0], acc[i][0]);
        acc[i][1] = __builtin_fmaf(p, vv[1], acc[i][1]);
        acc[i][2] = __builtin_fmaf(p, vv[2], acc[i][2]);
        acc[i][3] = __builtin_fmaf(p, vv[3], acc[i][3]);
      }
    }
    __syncthreads();
  }

  if (qvalid) {
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      *reinterpret_cast<f32x4*>(o + (head_q + qrow) * D + 16 * i + 4 * quad_lane) = acc[i] * inv;
    if (quad_lane == 0) lse[head_q + qrow] = (m_run + log2_fast(l_run)) * 0.69314718055994531f;
  }
}

template <int D>
hipError_t launch_d(const FwdArgs& a) {
  const int n_qtiles = (a.N + kF32Rows - 1) / kF32Rows;
  const uint64_t grid = (uint64_t)n_qtiles * a.Hq * a.B;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D>), dim3((uint32_t)grid), dim3(kF32Threads), 0,
                     a.stream, static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, a.Hq,
                     a.Hkv, a.N, a.scale * 1.44269504088896341f, n_qtiles, (uint32_t)a.n_xcd);
  return hipGetLastError();
}

}  // namespace

uint64_t fwd_f32_grid(int B, int Hq, int N) {
  return (uint64_t)((N + kF32Rows - 1) / kF32Rows) * Hq * B;
}

hipError_t launch_fwd_f32(const FwdArgs& a) {
  return a.d == 128 ? launch_d<128>(a) : launch_d<64>(a);
}

}  // namespace attn
