// attn_fwd_bf16.hip -- fused, tiled attention forward for gfx950, bf16 I/O.
//
// The IO-aware forward (blog "attention 的显存线性化", section 三; the
// "efficient attention" chapter's online-softmax paragraph): one workgroup
// owns kBr query rows of one head and streams every key/value tile of that
// head through LDS, keeping per row a running maximum m and exp-sum l and
// an fp32 output accumulator.  S and P only ever exist in registers.
//
// Design for CDNA4:
//  * 4 waves x 32 query rows.  Each wave computes S^T = K Q^T per 32-key
//    block with v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, the
//    wave's Q rows resident in VGPRs as the B operand).  In that output
//    layout a lane owns ONE query (column l % 32) and 16 of the 32 keys, so
//    the row max / row sum are in-lane reductions plus one exchange with
//    lane l ^ 32.
//  * O^T = V^T P^T on the same MFMA: P^T comes straight from the S^T
//    accumulator registers (rounded to bf16), V^T from LDS, and the O^T
//    accumulator again gives each lane one query, so the rescale by
//    exp(m_old - m_new) is a per-lane scalar.
//  * K tiles are staged row-major, V tiles transposed (V^T, keys fastest),
//    both padded so the MFMA-operand reads and the staging writes are free
//    of LDS bank conflicts; two stages, the next tile's global loads in
//    flight while the current tile is computed.
//  * The scale is folded into exp2: p = 2^(s * scale * log2 e - m).  The
//    running max is only moved when some row's max grows by more than
//    kRescaleLog2 (softmax is unchanged by any common shift of a row, the
//    basis of the rescale rule), so the rescale of the accumulator is rare.
//  * Workgroups of one K/V head are numbered consecutively and remapped so
//    they run on one XCD and share its L2.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bf16_tiles.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr float kRescaleLog2 = 8.0f;   // move m only when it grows by > 2^8

template <int D, bool kNegScale>
__global__ __launch_bounds__(kThreads, 2)
void attn_fwd_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                          const __bf16* __restrict__ v, __bf16* __restrict__ o,
                          float* __restrict__ lse, int Hq, int Hkv, int N, float c_log2,
                          int n_qtiles, uint32_t n_xcd) {
  using G = Geo<D>;
  __shared__ __align__(16) __bf16 smem[2 * G::kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- which (b, head, query tile) this workgroup owns -------------------
  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x, n_xcd);
  const int qt = (int)(logical % (uint32_t)n_qtiles);
  uint32_t rest = logical / (uint32_t)n_qtiles;
  const int group = Hq / Hkv;
  const int hg = (int)(rest % (uint32_t)group);
  rest /= (uint32_t)group;
  const int kvh = (int)(rest % (uint32_t)Hkv);
  const int b = (int)(rest / (uint32_t)Hkv);
  const int h = kvh * group + hg;

  const int64_t head_q = ((int64_t)b * Hq + h) * (int64_t)N;     // row index base
  const int64_t head_kv = ((int64_t)b * Hkv + kvh) * (int64_t)N;
  const __bf16* kh = k + head_kv * D;
  const __bf16* vh = v + head_kv * D;

  const int qrow = qt * kBr + wave * kRowsPerWave + l32;   // this lane's query
  const bool qvalid = qrow < N;

  // ---- Q^T fragments: lane holds d = 16 s + 8 hh .. +7 of its query -------
  bf16x8 qf[G::kKSteps];
  {
    const __bf16* qp = q + (head_q + (qvalid ? qrow : 0)) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < G::kKSteps; ++s) {
      u32x4 u = qvalid ? *reinterpret_cast<const u32x4*>(qp + 16 * s) : u32x4{0u, 0u, 0u, 0u};
      qf[s] = as_bf16x8(u);
    }
  }

  f32x16 oacc[G::kDB];
#pragma unroll
  for (int i = 0; i < G::kDB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;   // running max of the log2-scaled scores
  float l_run = 0.0f;        // this lane's part of the exp-sum (its 16 keys per block)

  const int n_tiles = (N + G::kBc - 1) / G::kBc;
  Regs regs;
  load_tile<D>(regs, kh, vh, 0, N, tid);
  store_tile<D>(regs, smem, smem + G::kKElems, tid);
  __syncthreads();

  for (int jt = 0; jt < n_tiles; ++jt) {
    const bool has_next = jt + 1 < n_tiles;
    if (has_next) load_tile<D>(regs, kh, vh, (jt + 1) * G::kBc, N, tid);

    const __bf16* ks = smem + (jt & 1) * G::kStage;
    const __bf16* vts = ks + G::kKElems;

    // ---- S^T = K Q^T for kKB blocks of 32 keys ---------------------------
    f32x16 sacc[G::kKB];
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb) {
      sacc[kb] = f32x16{};
      const __bf16* kr = ks + (kb * 32 + l32) * G::kKStr + 8 * hh;
#pragma unroll
      for (int s = 0; s < G::kKSteps; ++s) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(kr + 16 * s));
        sacc[kb] = mfma32x32x16(a, qf[s], sacc[kb]);
      }
    }

    // ---- online softmax on this lane's 16 * kKB scores -------------------
    const int j0 = jt * G::kBc;
    const bool tail = j0 + G::kBc > N;
    float ext;
    if (!tail) {
      ext = kNegScale ? INFINITY : -INFINITY;
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          ext = kNegScale ? fminf(ext, sacc[kb][e]) : fmaxf(ext, sacc[kb][e]);
      ext = kNegScale ? fminf(ext, __shfl_xor(ext, 32)) : fmaxf(ext, __shfl_xor(ext, 32));
      ext *= c_log2;   // max over the row of s * c_log2
    } else {
      // scale first, then mask keys >= N with -inf
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = j0 + kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
          sacc[kb][e] = key < N ? sacc[kb][e] * c_log2 : -INFINITY;
        }
      ext = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) ext = fmaxf(ext, sacc[kb][e]);
      ext = fmaxf(ext, __shfl_xor(ext, 32));
    }

    // move the running max only when some row's max grows by > 2^kRescaleLog2
    if (__any(ext > m_run + kRescaleLog2)) {
      const float m_new = fmaxf(m_run, ext);
      const float alpha = exp2_fast(m_run - m_new);   // 0 on the first tile
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < G::kDB; ++i) oacc[i] *= alpha;
    }

    bf16x8 pf[G::kKB][2];
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb) {
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = tail ? exp2_fast(sacc[kb][e] - m_run)
                    : exp2_fast(__builtin_fmaf(sacc[kb][e], c_log2, -m_run));
        lsum += p[e];
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 u;
#pragma unroll
        for (int w = 0; w < 4; ++w) u[w] = pack_bf16x2(p[8 * s2 + 2 * w], p[8 * s2 + 2 * w + 1]);
        pf[kb][s2] = as_bf16x8(u);
      }
    }
    l_run += lsum;

    // ---- O^T += V^T P^T ---------------------------------------------------
    // P^T slot (hh, e) of k-step s2 in block kb holds key kb*32 + 16 s2 +
    // 8 (e / 4) + 4 hh + e % 4; the V^T operand reads the same keys.
#pragma unroll
    for (int db = 0; db < G::kDB; ++db) {
      const __bf16* vr = vts + (db * 32 + l32) * G::kVStr + 4 * hh;
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int off = kb * 32 + 16 * s2;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vr + off);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + off + 8);
          const u32x4 u = {lo[0], lo[1], hi[0], hi[1]};
          oacc[db] = mfma32x32x16(as_bf16x8(u), pf[kb][s2], oacc[db]);
        }
    }

    if (has_next) store_tile<D>(regs, smem + ((jt + 1) & 1) * G::kStage,
                                smem + ((jt + 1) & 1) * G::kStage + G::kKElems, tid);
    __syncthreads();
  }

  // ---- epilogue: O = O~ / l, lse = (m + log2 l) ln 2 ------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qvalid) {
    const float inv = 1.0f / l_tot;
    __bf16* orow = o + (head_q + qrow) * D;
#pragma unroll
    for (int db = 0; db < G::kDB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * r + 0] * inv, oacc[db][4 * r + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * r + 2] * inv, oacc[db][4 * r + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * r + 4 * hh) = w;
      }
    if (hh == 0) lse[head_q + qrow] = (m_run + log2_fast(l_tot)) * 0.69314718055994531f;
  }
}

template <int D, bool kNeg>
hipError_t launch_d(const FwdArgs& a) {
  const int n_qtiles = (a.N + kBr - 1) / kBr;
  const uint64_t grid = (uint64_t)n_qtiles * a.Hq * a.B;
  const float c_log2 = a.scale * 1.44269504088896341f;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, kNeg>), dim3((uint32_t)grid), dim3(kThreads),
                     0, a.stream, static_cast<const __bf16*>(a.q),
                     static_cast<const __bf16*>(a.k), static_cast<const __bf16*>(a.v),
                     static_cast<__bf16*>(a.o), a.lse, a.Hq, a.Hkv, a.N, c_log2, n_qtiles,
                     (uint32_t)a.n_xcd);
  return hipGetLastError();
}

}  // namespace

uint64_t fwd_bf16_grid(int B, int Hq, int N) {
  return (uint64_t)((N + kBr - 1) / kBr) * Hq * B;
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  const bool neg = a.scale < 0.0f;
  if (a.d == 128) return neg ? launch_d<128, true>(a) : launch_d<128, false>(a);
  return neg ? launch_d<64, true>(a) : launch_d<64, false>(a);
}

}  // namespace attn
