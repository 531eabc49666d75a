// attn_materialized.hip -- the "standard attention" comparison path.
//
// Three kernels, each a full device-memory round trip of an [N, N] matrix
// per head, as the pages describe the unfused computation (aiknowledge.cn
// "1.1 注意力计算的计算与显存瓶颈", sections 1.1.1 and 1.1.3: write S, read
// S back for the row softmax, write P, read P back to multiply by V):
//   qk kernel       S = scale * Q K^T                  -> s  (fp32)
//   softmax kernel  P = row softmax of S, lse per row  -> p  (I/O dtype), lse
//   pv kernel       O = P V                            -> o  (I/O dtype)
// bf16: both products on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
// fp32: plain vector FMA in fp32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bf16_tiles.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

// ---------------------------------------------------------------------------
// S = scale * Q K^T, bf16 inputs, one workgroup per 128 x 128 block of S.
// Wave w computes queries [qt*128 + 32 w, +32) x keys [kt*128, +128) as four
// 32 x 32 S blocks (Q as the A operand in VGPRs, K^T as the B operand read
// straight from global memory).
template <int D>
__global__ __launch_bounds__(kThreads)
void qk_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                    float* __restrict__ s, int Hq, int Hkv, int N, float scale, int n_t) {
  constexpr int kSteps = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int kt = blockIdx.x % n_t;
  const int qt = (blockIdx.x / n_t) % n_t;
  const int bh = blockIdx.x / (n_t * n_t);
  const int b = bh / Hq, h = bh % Hq;
  const int kvh = h / (Hq / Hkv);
  const __bf16* qh = q + ((int64_t)b * Hq + h) * N * D;
  const __bf16* kh = k + ((int64_t)b * Hkv + kvh) * N * D;
  float* sh = s + ((int64_t)b * Hq + h) * N * (int64_t)N;

  const int qrow = qt * 128 + wave * 32 + l32;
  bf16x8 qf[kSteps];
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    u32x4 u = qrow < N ? *reinterpret_cast<const u32x4*>(qh + (int64_t)qrow * D + 16 * st + 8 * hh)
                       : u32x4{0u, 0u, 0u, 0u};
    qf[st] = as_bf16x8(u);
  }
  // All four key blocks' K operands are loaded before the first product,
  // and S (not S^T) is accumulated: with Q as the A operand a lane holds one
  // key of 16 queries, so each store writes 128 contiguous bytes of two rows.
  bf16x8 kf[4][kSteps];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int krow = kt * 128 + kb * 32 + l32;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      u32x4 u = krow < N ? *reinterpret_cast<const u32x4*>(kh + (int64_t)krow * D + 16 * st + 8 * hh)
                         : u32x4{0u, 0u, 0u, 0u};
      kf[kb][st] = as_bf16x8(u);
    }
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int key = kt * 128 + kb * 32 + l32;          // this lane's key
    f32x16 acc = f32x16{};
#pragma unroll
    for (int st = 0; st < kSteps; ++st) acc = mfma32x32x16(qf[st], kf[kb][st], acc);
    // element 4 r + t of a lane is S[query 8 r + 4 hh + t of the wave][key]
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int qr = qt * 128 + wave * 32 + 8 * r + 4 * hh + t;
        if (qr < N && key < N) sh[(int64_t)qr * N + key] = acc[4 * r + t] * scale;
      }
  }
}

// ---------------------------------------------------------------------------
// Row softmax of S: one workgroup per row.  Pass 1 keeps a per-thread
// (max, exp-sum) over a strided part of the row, merged across the
// workgroup; pass 2 re-reads the row (now in L2) and writes
// P = exp(S - m) / l in the output type.  lse = m + ln l.
template <typename OutT>
__device__ __forceinline__ void store_p(OutT* p, int64_t i, float x);
template <>
__device__ __forceinline__ void store_p<float>(float* p, int64_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void store_p<__bf16>(__bf16* p, int64_t i, float x) { p[i] = (__bf16)x; }

__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;   // both empty
  l = l * exp2_fast((m - mn) * 1.44269504088896341f) + l2 * exp2_fast((m2 - mn) * 1.44269504088896341f);
  m = mn;
}

template <typename OutT>
__global__ __launch_bounds__(256)
void softmax_rows_kernel(const float* __restrict__ s, OutT* __restrict__ p, float* __restrict__ lse,
                         int N) {
  __shared__ float red_m[4], red_l[4];
  const int64_t row = blockIdx.x;
  const float* srow = s + row * (int64_t)N;
  const int tid = threadIdx.x;
  constexpr float kL2e = 1.44269504088896341f;

  float m = -INFINITY, l = 0.0f;
  for (int j = tid; j < N; j += 256) {
    const float x = srow[j];
    if (x > m) {
      l = l * exp2_fast((m - x) * kL2e) + 1.0f;
      m = x;
    } else {
      l += exp2_fast((x - m) * kL2e);
    }
  }
  // wave reduction, then across the four waves
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    merge_ml(m, l, m2, l2);
  }
  if ((tid & 63) == 0) {
    red_m[tid >> 6] = m;
    red_l[tid >> 6] = l;
  }
  __syncthreads();
  m = red_m[0];
  l = red_l[0];
  for (int w = 1; w < 4; ++w) merge_ml(m, l, red_m[w], red_l[w]);

  const float inv = 1.0f / l;
  OutT* prow = p + row * (int64_t)N;
  for (int j = tid; j < N; j += 256) store_p<OutT>(prow, j, exp2_fast((srow[j] - m) * kL2e) * inv);
  if (tid == 0) lse[row] = m + logf(l);
}

// The same with 16-byte accesses (rows of N % 4 == 0 floats are 16-byte
// aligned): each thread takes whole 4-score chunks, keeping (max, exp-sum)
// per chunk rather than per score, and writes its 4 weights at once.
template <typename OutT>
__device__ __forceinline__ void store_p4(OutT* p, int64_t i, f32x4 x);
template <>
__device__ __forceinline__ void store_p4<float>(float* p, int64_t i, f32x4 x) {
  *reinterpret_cast<f32x4*>(p + i) = x;
}
template <>
__device__ __forceinline__ void store_p4<__bf16>(__bf16* p, int64_t i, f32x4 x) {
  u32x2 w;
  w[0] = pack_bf16x2(x[0], x[1]);
  w[1] = pack_bf16x2(x[2], x[3]);
  *reinterpret_cast<u32x2*>(p + i) = w;
}

template <typename OutT>
__global__ __launch_bounds__(256)
void softmax_rows_vec_kernel(const float* __restrict__ s, OutT* __restrict__ p,
                             float* __restrict__ lse, int N) {
  __shared__ float red_m[4], red_l[4];
  const int64_t row = blockIdx.x;
  const float* srow = s + row * (int64_t)N;
  const int tid = threadIdx.x;
  const int n4 = N / 4;
  constexpr float kL2e = 1.44269504088896341f;

  float m = -INFINITY, l = 0.0f;
  for (int j = tid; j < n4; j += 256) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(srow + 4 * j);
    const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    const float mn = fmaxf(m, mx);
    const float part = exp2_fast((x[0] - mn) * kL2e) + exp2_fast((x[1] - mn) * kL2e) +
                       exp2_fast((x[2] - mn) * kL2e) + exp2_fast((x[3] - mn) * kL2e);
    l = (m == -INFINITY ? 0.0f : l * exp2_fast((m - mn) * kL2e)) + part;
    m = mn;
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    merge_ml(m, l, m2, l2);
  }
  if ((tid & 63) == 0) {
    red_m[tid >> 6] = m;
    red_l[tid >> 6] = l;
  }
  __syncthreads();
  m = red_m[0];
  l = red_l[0];
  for (int w = 1; w < 4; ++w) merge_ml(m, l, red_m[w], red_l[w]);

  const float inv = 1.0f / l;
  OutT* prow = p + row * (int64_t)N;
  for (int j = tid; j < n4; j += 256) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(srow + 4 * j);
    f32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = exp2_fast((x[i] - m) * kL2e) * inv;
    store_p4<OutT>(prow, 4 * (int64_t)j, y);
  }
  if (tid == 0) lse[row] = m + logf(l);
}

// Rows of at most kWaveRowMax scores (N % 4 == 0): one wave per row, the
// row held in registers (16-byte loads, up to 16 per lane), so S is read
// from memory once; max and exp-sum by wave reductions.
constexpr int kWaveRowChunks = 16;                       // 4-score chunks per lane
constexpr int kWaveRowMax = kWaveRowChunks * 4 * kWave;  // 4096 scores

template <typename OutT>
__global__ __launch_bounds__(256)
void softmax_rows_wave_kernel(const float* __restrict__ s, OutT* __restrict__ p,
                              float* __restrict__ lse, int N, int64_t n_rows) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const float* srow = s + row * (int64_t)N;
  constexpr float kL2e = 1.44269504088896341f;
  const int n4 = N / 4;

  f32x4 x[kWaveRowChunks];
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < kWaveRowChunks; ++c) {
    const int j = c * kWave + lane;
    if (j < n4) {
      x[c] = *reinterpret_cast<const f32x4*>(srow + 4 * j);
      m = fmaxf(m, fmaxf(fmaxf(x[c][0], x[c][1]), fmaxf(x[c][2], x[c][3])));
    }
  }
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float l = 0.0f;
#pragma unroll
  for (int c = 0; c < kWaveRowChunks; ++c) {
    if (c * kWave + lane < n4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[c][i] = exp2_fast((x[c][i] - m) * kL2e);
        l += x[c][i];
      }
    }
  }
  for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
  const float inv = 1.0f / l;
  OutT* prow = p + row * (int64_t)N;
#pragma unroll
  for (int c = 0; c < kWaveRowChunks; ++c) {
    const int j = c * kWave + lane;
    if (j < n4) store_p4<OutT>(prow, 4 * (int64_t)j, x[c] * inv);
  }
  if (lane == 0) lse[row] = m + logf(l);
}

// ---------------------------------------------------------------------------
// O = P V, bf16: one workgroup per 128 query rows of a head.  V tiles are
// staged transposed through LDS (shared staging with the fused kernel); P^T
// operands are read straight from global memory, 16 bytes per lane when the
// rows are 16-byte aligned.  O^T = V^T P^T accumulates in fp32; lane
// (query l%32, half h) ends with d = 32 db + 8 r + 4 h + {0..3}.
template <int D, bool kVecP>
__global__ __launch_bounds__(kThreads, 2)
void pv_bf16_kernel(const __bf16* __restrict__ p, const __bf16* __restrict__ v,
                    __bf16* __restrict__ o, int Hq, int Hkv, int N, int n_qtiles) {
  using G = Geo<D>;
  __shared__ __align__(16) __bf16 vts[G::kVElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int qt = blockIdx.x % n_qtiles;
  const int bh = blockIdx.x / n_qtiles;
  const int b = bh / Hq, h = bh % Hq;
  const int kvh = h / (Hq / Hkv);
  const __bf16* vh = v + ((int64_t)b * Hkv + kvh) * N * D;
  const __bf16* ph = p + ((int64_t)b * Hq + h) * N * (int64_t)N;
  const int qrow = qt * kBr + wave * kRowsPerWave + l32;
  const bool qvalid = qrow < N;
  const __bf16* prow = ph + (int64_t)(qvalid ? qrow : 0) * N;

  f32x16 oacc[G::kDB];
#pragma unroll
  for (int i = 0; i < G::kDB; ++i) oacc[i] = f32x16{};

  // P^T fragments of one tile: slot (hh, e) of k-step s2 in block kb is key
  // j0 + kb * 32 + 16 s2 + 8 hh + e of this lane's row
  auto load_p = [&](u32x4 (&pu)[G::kKB][2], int j0) {
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int key0 = j0 + kb * 32 + 16 * s2 + 8 * hh;
        if (kVecP && qvalid && key0 + 7 < N) {
          pu[kb][s2] = *reinterpret_cast<const u32x4*>(prow + key0);
        } else {
          uint16_t hw[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            hw[e] = (qvalid && key0 + e < N) ? reinterpret_cast<const uint16_t*>(prow)[key0 + e] : 0;
#pragma unroll
          for (int w = 0; w < 4; ++w)
            pu[kb][s2][w] = (uint32_t)hw[2 * w] | ((uint32_t)hw[2 * w + 1] << 16);
        }
      }
  };

  // The next tile's V (through registers) and P fragments are loaded while
  // the current tile's products run.
  const int n_tiles = (N + G::kBc - 1) / G::kBc;
  Regs regs;
  u32x4 pn[G::kKB][2];
  load_v_tile<D>(regs, vh, 0, N, tid);
  load_p(pn, 0);
  for (int jt = 0; jt < n_tiles; ++jt) {
    store_v_tile<D>(regs, vts, tid);
    __syncthreads();
    u32x4 pc[G::kKB][2];
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) pc[kb][s2] = pn[kb][s2];
    if (jt + 1 < n_tiles) {
      load_v_tile<D>(regs, vh, (jt + 1) * G::kBc, N, tid);
      load_p(pn, (jt + 1) * G::kBc);
    }
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 pf = as_bf16x8(pc[kb][s2]);
#pragma unroll
        for (int db = 0; db < G::kDB; ++db) {
          const __bf16* vr = vts + (db * 32 + l32) * G::kVStr + kb * 32 + 16 * s2 + 8 * hh;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 4);
          const u32x4 u = {lo[0], lo[1], hi[0], hi[1]};
          oacc[db] = mfma32x32x16(as_bf16x8(u), pf, oacc[db]);
        }
      }
    __syncthreads();
  }
  if (qvalid) {
    __bf16* orow = o + (((int64_t)b * Hq + h) * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < G::kDB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * r + 0], oacc[db][4 * r + 1]);
        w[1] = pack_bf16x2(oacc[db][4 * r + 2], oacc[db][4 * r + 3]);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * r + 4 * hh) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// fp32 products on the vector units.  S = scale * Q K^T: a workgroup of
// 16 x 16 threads computes a 64 x 64 block of S, 4 x 4 per thread, from Q and
// K tiles of 64 rows x 16 d staged in LDS.
constexpr int kGT = 64;   // tile edge
constexpr int kGK = 16;   // d slice per stage

__global__ __launch_bounds__(256)
void qk_f32_kernel(const float* __restrict__ q, const float* __restrict__ k, float* __restrict__ s,
                   int Hq, int Hkv, int N, int D, float scale, int n_t) {
  __shared__ float qs[kGK][kGT + 1];
  __shared__ float kss[kGK][kGT + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int kt = blockIdx.x % n_t;
  const int qt = (blockIdx.x / n_t) % n_t;
  const int bh = blockIdx.x / (n_t * n_t);
  const int b = bh / Hq, h = bh % Hq;
  const int kvh = h / (Hq / Hkv);
  const float* qh = q + ((int64_t)b * Hq + h) * N * D;
  const float* kh = k + ((int64_t)b * Hkv + kvh) * N * D;
  float acc[4][4] = {};
  for (int c0 = 0; c0 < D; c0 += kGK) {
    for (int e = threadIdx.x; e < kGT * kGK; e += 256) {
      const int r = e / kGK, c = e % kGK;
      const int qi = qt * kGT + r, kj = kt * kGT + r;
      qs[c][r] = qi < N ? qh[(int64_t)qi * D + c0 + c] : 0.0f;
      kss[c][r] = kj < N ? kh[(int64_t)kj * D + c0 + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kGK; ++c) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = qs[c][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = kss[c][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* sh = s + ((int64_t)b * Hq + h) * N * (int64_t)N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qi = qt * kGT + ty + 16 * i;
    if (qi >= N) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kj = kt * kGT + tx + 16 * j;
      if (kj < N) sh[(int64_t)qi * N + kj] = acc[i][j] * scale;
    }
  }
}

// O = P V in fp32: a workgroup computes 64 query rows x D columns; thread
// (ty, tx) of 16 x 16 owns rows ty + 16 i and columns tx + 16 j.
template <int D>
__global__ __launch_bounds__(256)
void pv_f32_kernel(const float* __restrict__ p, const float* __restrict__ v, float* __restrict__ o,
                   int Hq, int Hkv, int N, int n_qt) {
  constexpr int kCols = D / 16;
  __shared__ float ps[kGK][kGT + 1];
  __shared__ float vs[kGK][D];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int qt = blockIdx.x % n_qt;
  const int bh = blockIdx.x / n_qt;
  const int b = bh / Hq, h = bh % Hq;
  const int kvh = h / (Hq / Hkv);
  const float* ph = p + ((int64_t)b * Hq + h) * N * (int64_t)N;
  const float* vh = v + ((int64_t)b * Hkv + kvh) * N * D;
  float acc[4][kCols] = {};
  for (int j0 = 0; j0 < N; j0 += kGK) {
    for (int e = threadIdx.x; e < kGT * kGK; e += 256) {
      const int r = e / kGK, c = e % kGK;
      const int qi = qt * kGT + r, kj = j0 + c;
      ps[c][r] = (qi < N && kj < N) ? ph[(int64_t)qi * N + kj] : 0.0f;
    }
    for (int e = threadIdx.x; e < kGK * D; e += 256) {
      const int r = e / D, c = e % D;
      vs[r][c] = (j0 + r < N) ? vh[(int64_t)(j0 + r) * D + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < kGK; ++jj) {
      float a[4], bb[kCols];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = ps[jj][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < kCols; ++j) bb[j] = vs[jj][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kCols; ++j) acc[i][j] = __builtin_fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qi = qt * kGT + ty + 16 * i;
    if (qi >= N) continue;
    float* orow = o + (((int64_t)b * Hq + h) * N + qi) * D;
#pragma unroll
    for (int j = 0; j < kCols; ++j) orow[tx + 16 * j] = acc[i][j];
  }
}

template <int D>
hipError_t launch_bf16_d(const FwdArgs& a) {
  const int n_t = (a.N + 127) / 128;
  const uint64_t rows = (uint64_t)a.B * a.Hq * a.N;
  hipLaunchKernelGGL((qk_bf16_kernel<D>), dim3((uint32_t)((uint64_t)n_t * n_t * a.B * a.Hq)),
                     dim3(kThreads), 0, a.stream, static_cast<const __bf16*>(a.q),
                     static_cast<const __bf16*>(a.k), a.s, a.Hq, a.Hkv, a.N, a.scale, n_t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.N % 4 == 0 && a.N <= kWaveRowMax)
    hipLaunchKernelGGL((softmax_rows_wave_kernel<__bf16>), dim3((uint32_t)((rows + 3) / 4)),
                       dim3(256), 0, a.stream, a.s, static_cast<__bf16*>(a.p), a.lse, a.N,
                       (int64_t)rows);
  else if (a.N % 4 == 0)
    hipLaunchKernelGGL((softmax_rows_vec_kernel<__bf16>), dim3((uint32_t)rows), dim3(256), 0,
                       a.stream, a.s, static_cast<__bf16*>(a.p), a.lse, a.N);
  else
    hipLaunchKernelGGL((softmax_rows_kernel<__bf16>), dim3((uint32_t)rows), dim3(256), 0, a.stream,
                       a.s, static_cast<__bf16*>(a.p), a.lse, a.N);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_qt = (a.N + kBr - 1) / kBr;
  const dim3 grid((uint32_t)((uint64_t)n_qt * a.B * a.Hq));
  if (a.N % 8 == 0) {
    hipLaunchKernelGGL((pv_bf16_kernel<D, true>), grid, dim3(kThreads), 0, a.stream,
                       static_cast<const __bf16*>(a.p), static_cast<const __bf16*>(a.v),
                       static_cast<__bf16*>(a.o), a.Hq, a.Hkv, a.N, n_qt);
  } else {
    hipLaunchKernelGGL((pv_bf16_kernel<D, false>), grid, dim3(kThreads), 0, a.stream,
                       static_cast<const __bf16*>(a.p), static_cast<const __bf16*>(a.v),
                       static_cast<__bf16*>(a.o), a.Hq, a.Hkv, a.N, n_qt);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32_d(const FwdArgs& a) {
  const int n_t = (a.N + kGT - 1) / kGT;
  const uint64_t rows = (uint64_t)a.B * a.Hq * a.N;
  hipLaunchKernelGGL(qk_f32_kernel, dim3((uint32_t)((uint64_t)n_t * n_t * a.B * a.Hq)), dim3(256),
                     0, a.stream, static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     a.s, a.Hq, a.Hkv, a.N, D, a.scale, n_t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.N % 4 == 0 && a.N <= kWaveRowMax)
    hipLaunchKernelGGL((softmax_rows_wave_kernel<float>), dim3((uint32_t)((rows + 3) / 4)),
                       dim3(256), 0, a.stream, a.s, static_cast<float*>(a.p), a.lse, a.N,
                       (int64_t)rows);
  else if (a.N % 4 == 0)
    hipLaunchKernelGGL((softmax_rows_vec_kernel<float>), dim3((uint32_t)rows), dim3(256), 0,
                       a.stream, a.s, static_cast<float*>(a.p), a.lse, a.N);
  else
    hipLaunchKernelGGL((softmax_rows_kernel<float>), dim3((uint32_t)rows), dim3(256), 0, a.stream,
                       a.s, static_cast<float*>(a.p), a.lse, a.N);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((pv_f32_kernel<D>), dim3((uint32_t)((uint64_t)n_t * a.B * a.Hq)), dim3(256), 0,
                     a.stream, static_cast<const float*>(a.p), static_cast<const float*>(a.v),
                     static_cast<float*>(a.o), a.Hq, a.Hkv, a.N, n_t);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_materialized_bf16(const FwdArgs& a) {
  return a.d == 128 ? launch_bf16_d<128>(a) : launch_bf16_d<64>(a);
}

hipError_t launch_materialized_f32(const FwdArgs& a) {
  return a.d == 128 ? launch_f32_d<128>(a) : launch_f32_d<64>(a);
}

}  // namespace attn
