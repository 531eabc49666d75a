// attn_fwd_fp8.hip -- fused, tiled attention forward for gfx950 with 8-bit
// floating-point inputs (OCP E4M3) on the FP8 matrix cores.
//
// The IO-aware forward (blog "attention 的显存线性化", section 三; the
// "efficient attention" chapter's online-softmax paragraph), in the 8-bit
// form the pages name for the third FlashAttention version without its
// arithmetic (same blog, section 五).  Both products run on
// v_mfma_f32_32x32x64_f8f6f4 (E4M3 operands, fp32 accumulation), at twice
// the bf16 rate per instruction byte.
//
// Inputs: q8 [B,Hq,N,d], k8 [B,Hkv,N,d] and vt8 = V transposed,
// [B,Hkv,d,Np] (Np = N rounded up to 16), E4M3 codes, with one float scale
// per tensor; the scores' scale and the q / k scales are folded into the
// exponent's multiplier, the v scale into the final division.
//
// What differs from the bf16 rows32 kernel it follows:
//  * S^T = K Q^T: 32-key blocks, k-steps of 64 bytes of d; a lane of half h
//    supplies bytes 32 h .. 32 h + 31 of its row to each k-step, for the K
//    rows (A, from LDS) and its Q row (B, in VGPRs) alike, so the slots of
//    the two operands name the same d.
//  * The weights are rounded to E4M3 for the PV product after a 2^6 scale
//    (a weight equal to e^(running max) becomes 64; the running max moves
//    when a row max grows by more than 2^2, so weights stay <= 2^8 < 448);
//    the exp-sum adds the unrounded fp32 weights.
//  * P^T as the B operand of O^T = V^T P^T needs one lane half to hold keys
//    0..31 of the 64-key tile and the other 32..63, each in key order; the
//    S accumulator gives a lane 4-key runs of both 32-key blocks, so one
//    v_permlane32_swap per pair of packed runs regroups them.  V^T comes
//    from the transposed input: a lane reads 32 consecutive keys of its d
//    row, two 16-byte LDS reads, no transposing read needed.
//  * Keys N .. of the last tile: K rows read as zeros (buffer range) and
//    their weights are set to 0; the V^T bytes of those keys (padding or the
//    next row) are cleared in registers, so no NaN code reaches the MFMA.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRows = 32;                  // query rows per wave
constexpr int kBr = kWaves * kRows;        // query rows per workgroup
constexpr int kBc = 64;                    // keys per tile
constexpr float kRescaleLog2 = 2.0f;       // move m only when a row max grows by > 2^2
constexpr float kPScaleLog2 = 6.0f;        // weights scaled by 2^6 before rounding to E4M3

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int D>
struct G8 {
  static constexpr int kKSteps = D / 64;                  // k-steps over d
  static constexpr int kDB = D / 32;                      // 32-wide d blocks of O
  static constexpr int kTileB = kBc * D;                  // bytes of a K tile (= a V^T tile)
  static constexpr int kStageB = 2 * kTileB;              // K tile, then V^T tile
  static constexpr int kKCpr = D / 16;                    // 16-byte chunks per K row
  static constexpr int kDma = kTileB / 16 / kThreads;     // 16-byte loads per lane per tile
  static_assert(kDma * 16 * kThreads == kTileB, "tile must split over the workgroup");
};

// Chunk swizzles (16-byte chunk c of row r stored at c ^ swz(r)), so that the
// 16 lanes of one LDS read -- one chunk of 16 consecutive rows -- hit 16
// distinct 16-byte bank groups of the 256-byte bank space:
//  * 128-byte rows (K at d = 128): rows 2m and 2m + 1 share a 256-byte
//    line, the 8 pairs get distinct chunks;
//  * 64-byte rows (K at d = 64, every V^T tile): 4 rows per line, the 4
//    lines get distinct chunks.
template <int RowB>
__device__ __forceinline__ int swz8(int row) {
  return RowB == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

__device__ __forceinline__ int srows(int rem, int hi) {
  int r;
  asm("s_max_i32 %0, %1, 0\n\ts_min_i32 %0, %0, %2" : "=&s"(r) : "s"(rem), "s"(hi) : "scc");
  return r;
}

// Direct global -> LDS loads of one tile: instruction i of this wave fills
// LDS chunks (wave * kDma + i) * 64 + lane, lane's source byte offset
// within the buffer being off[i].  Inline assembly, as in the bf16 kernels,
// so the compiler does not hold LDS reads of the other stage behind it.
template <int D>
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t rs, uint32_t lds_tile, int wave,
                                    const int* off) {
#pragma unroll
  for (int i = 0; i < G8<D>::kDma; ++i) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(
        lds_tile + (uint32_t)((wave * G8<D>::kDma + i) * kWave * 16));
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 ::"s"(dst), "v"(off[i]), "s"(rs) : "memory");
  }
}

// K rows j0 .. j0 + 63 of a head: the buffer covers rows j0 .. N-1 only.
template <int D>
__device__ __forceinline__ void dma_k(const uint8_t* head, int j0, int N, uint32_t lds_tile,
                                      int wave, const int* off) {
  const int rows = srows(N - j0, kBc);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(head) + (int64_t)min(j0, N) * D, (short)0, rows * D, 0x00020000);
  dma<D>(rs, lds_tile, wave, off);
}

// V^T columns j0 .. j0 + 63 of the D rows of a head (row length Np bytes):
// the buffer starts at column j0 and ends with the head, so nothing past the
// head is read; columns past N within it are cleared after the LDS read.
template <int D>
__device__ __forceinline__ void dma_vt(const uint8_t* head, int j0, int Np, uint32_t lds_tile,
                                       int wave, const int* off) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(head) + j0, (short)0, D * Np - j0, 0x00020000);
  dma<D>(rs, lds_tile, wave, off);
}

__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmin(float a, float b) { return __builtin_elementwise_minimum(a, b); }

__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_min(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmin(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // format codes 0 / 0: both operands E4M3; no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four fp32 values rounded to E4M3 (nearest even) and packed in order,
// the first in the low byte.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ i32x8 lds_read32(const uint8_t* p0, const uint8_t* p1) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p0);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(p1);
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Three workgroups per CU at d = 128 (168 VGPRs; 7 % faster than two),
// four at d = 64.
template <int D, bool kNegScale>
__global__ __launch_bounds__(kThreads, D == 64 ? 4 : 3)
void attn_fwd_fp8_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                         const uint8_t* __restrict__ vt, __bf16* __restrict__ o,
                         float* __restrict__ lse, int Hq, int Hkv, int N, int Np, float c_log2,
                         float v_scale, int n_qtiles, uint32_t n_xcd) {
  using G = G8<D>;
  __shared__ __align__(16) uint8_t smem[2 * G::kStageB];
  const uint32_t lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // direct-load source offsets: LDS chunk g = slot + lane holds logical
  // chunk (g % cpr) ^ swz(row) of row g / cpr
  int koff_dma[G::kDma], voff_dma[G::kDma];
#pragma unroll
  for (int i = 0; i < G::kDma; ++i) {
    const int g = (wave * G::kDma + i) * kWave + lane;
    const int kr = g / G::kKCpr;
    koff_dma[i] = kr * D + (((g % G::kKCpr) ^ swz8<D>(kr)) * 16);
    const int vr = g / 4;
    voff_dma[i] = vr * Np + (((g % 4) ^ swz8<64>(vr)) * 16);
  }

  // ---- which (b, K/V head, query tile): query tiles over the group's
  // (Hq / Hkv) * N adjacent rows, numbered fastest (as the bf16 kernels)
  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x, n_xcd);
  const int qt = (int)(logical % (uint32_t)n_qtiles);
  const uint32_t rest = logical / (uint32_t)n_qtiles;
  const int kvh = (int)(rest % (uint32_t)Hkv);
  const int b = (int)(rest / (uint32_t)Hkv);
  const int n_qrows = (Hq / Hkv) * N;
  const int64_t head_q = ((int64_t)b * Hkv + kvh) * (int64_t)n_qrows;
  const int64_t head_kv = (int64_t)b * Hkv + kvh;
  const uint8_t* kh = k + head_kv * (int64_t)N * D;
  const uint8_t* vh = vt + head_kv * (int64_t)D * Np;

  const int n_tiles = (N + kBc - 1) / kBc;
  dma_k<D>(kh, 0, N, lds, wave, koff_dma);
  dma_vt<D>(vh, 0, Np, lds + G::kTileB, wave, voff_dma);

  const int qrow = qt * kBr + wave * kRows + l32;
  const bool qvalid = qrow < n_qrows;

  // ---- Q fragments (B operand): bytes 64 s + 32 hh .. +31 of the query row
  i32x8 qf[G::kKSteps];
  {
    const uint8_t* qp = q + (head_q + (qvalid ? qrow : 0)) * D + 32 * hh;
#pragma unroll
    for (int s = 0; s < G::kKSteps; ++s) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      const u32x4 lo = qvalid ? *reinterpret_cast<const u32x4*>(qp + 64 * s) : z;
      const u32x4 hi = qvalid ? *reinterpret_cast<const u32x4*>(qp + 64 * s + 16) : z;
      qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }

  // ---- LDS read offsets (bytes) ------------------------------------------
  // K (A operand of S^T): row kb * 32 + l32, chunks 4 s + 2 hh and + 1
  int kro[G::kKSteps][2];
#pragma unroll
  for (int s = 0; s < G::kKSteps; ++s)
#pragma unroll
    for (int e = 0; e < 2; ++e) kro[s][e] = l32 * D + (((4 * s + 2 * hh + e) ^ swz8<D>(l32)) * 16);
  // V^T (A operand of O^T): row db * 32 + l32, chunks 2 hh and + 1
  int vro[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) vro[e] = l32 * kBc + (((2 * hh + e) ^ swz8<64>(l32)) * 16);

  f32x16 oacc[G::kDB];
#pragma unroll
  for (int i = 0; i < G::kDB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;   // running max of the log2-scaled scores
  float l_run = 0.0f;        // this lane's part of the (2^6-scaled) exp-sum

  wait_dma();
  __syncthreads();

  // One key tile in LDS stage `stage` (a compile-time constant: the loop
  // below runs two tiles per trip, so every LDS read has a fixed offset).
  auto tile = [&](const int jt, auto stage_c) {
    constexpr int stage = decltype(stage_c)::value;
    const uint8_t* ks = smem + stage * G::kStageB;
    const uint8_t* vs = ks + G::kTileB;
    if (jt + 1 < n_tiles) {
      const uint32_t nxt = lds + (uint32_t)((1 - stage) * G::kStageB);
      dma_k<D>(kh, (jt + 1) * kBc, N, nxt, wave, koff_dma);
      dma_vt<D>(vh, (jt + 1) * kBc, Np, nxt + G::kTileB, wave, voff_dma);
    }

    // ---- S^T = K Q^T for two blocks of 32 keys ----------------------------
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < G::kKSteps; ++s) {
        const uint8_t* base = ks + kb * 32 * D;
        sacc[kb] = mfma_f8(lds_read32(base + kro[s][0], base + kro[s][1]), qf[s], sacc[kb]);
      }
    }

    // ---- online softmax on this lane's 32 scores ---------------------------
    const int j0 = jt * kBc;
    const bool tail = j0 + kBc > N;
    float ext;
    if (!tail) {
      float t[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x16& a = sacc[kb];
          t[kb * 4 + r] = kNegScale
              ? vmin(vmin(a[4 * r], a[4 * r + 1]), vmin(a[4 * r + 2], a[4 * r + 3]))
              : vmax(vmax(a[4 * r], a[4 * r + 1]), vmax(a[4 * r + 2], a[4 * r + 3]));
        }
#pragma unroll
      for (int w = 8; w > 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w / 2; ++i)
          t[i] = kNegScale ? vmin(t[i], t[i + w / 2]) : vmax(t[i], t[i + w / 2]);
      ext = t[0];
    } else {
      float e2 = kNegScale ? INFINITY : -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = j0 + kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
          if (key < N) e2 = kNegScale ? vmin(e2, sacc[kb][e]) : vmax(e2, sacc[kb][e]);
        }
      ext = e2;
    }

    // the test on each half-row's own max; both halves' max only on a move
    if (__builtin_amdgcn_ballot_w64(__builtin_fmaf(ext, c_log2, -m_run) > kRescaleLog2) != 0) {
      ext = (kNegScale ? xhalf_min(ext) : xhalf_max(ext)) * c_log2;
      const float m_new = fmaxf(m_run, ext);
      const float alpha = exp2_fast(m_run - m_new);   // 0 on the first tile
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < G::kDB; ++i) oacc[i] *= alpha;
    }

    const float msub = kPScaleLog2 - m_run;
    float p[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) p[kb][e] = exp2_fast(__builtin_fmaf(sacc[kb][e], c_log2, msub));
    if (tail) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = j0 + kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
          if (key >= N) p[kb][e] = 0.0f;
        }
    }
    {
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) ps[e & 3] += p[kb][e];
      l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }

    // ---- P^T operand: lane half 0 keys 0..31, half 1 keys 32..63 -----------
    // run r of block kb holds keys kb*32 + 8 r + 4 hh + 0..3; swapping run r
    // of block 0 (upper half) with run r of block 1 (lower half) leaves
    // half 0 with keys 8 r + 0..7 and half 1 with 32 + 8 r + 0..7.
    i32x8 pb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t x = pack_e4m3x4(p[0][4 * r], p[0][4 * r + 1], p[0][4 * r + 2], p[0][4 * r + 3]);
      const uint32_t y = pack_e4m3x4(p[1][4 * r], p[1][4 * r + 1], p[1][4 * r + 2], p[1][4 * r + 3]);
      const auto sw = __builtin_amdgcn_permlane32_swap(x, y, false, false);
      pb[2 * r] = (int)sw[0];
      pb[2 * r + 1] = (int)sw[1];
    }

    // ---- O^T += V^T P^T -----------------------------------------------------
    // byte mask of keys < N among this lane's 32 (keys j0 + 32 hh + 0..31)
    uint32_t vmask[8];
    if (tail) {
      const int nv = N - j0 - 32 * hh;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int nb = min(max(nv - 4 * w, 0), 4);
        vmask[w] = nb >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nb)) - 1u);
      }
    }
#pragma unroll
    for (int db = 0; db < G::kDB; ++db) {
      const uint8_t* base = vs + db * 32 * kBc;
      i32x8 a = lds_read32(base + vro[0], base + vro[1]);
      if (tail) {
#pragma unroll
        for (int w = 0; w < 8; ++w) a[w] = (int)((uint32_t)a[w] & vmask[w]);
      }
      oacc[db] = mfma_f8(a, pb, oacc[db]);
    }

    wait_dma();
    __syncthreads();
  };
  for (int jt = 0; jt < n_tiles; jt += 2) {
    tile(jt, std::integral_constant<int, 0>{});
    if (jt + 1 < n_tiles) tile(jt + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: O = v_scale * O~ / l, lse = (m + log2 l - 6) ln 2 ----------
  const float l_tot = xhalf_sum(l_run);
  if (qvalid) {
    const float mul = v_scale / l_tot;
    __bf16* orow = o + (head_q + qrow) * D;
#pragma unroll
    for (int db = 0; db < G::kDB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * r + 0] * mul, oacc[db][4 * r + 1] * mul);
        w[1] = pack_bf16x2(oacc[db][4 * r + 2] * mul, oacc[db][4 * r + 3] * mul);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * r + 4 * hh) = w;
      }
    if (hh == 0)
      lse[head_q + qrow] = (m_run - kPScaleLog2 + log2_fast(l_tot)) * 0.69314718055994531f;
  }
}

template <int D, bool kNeg>
hipError_t launch_d(const FwdArgs& a) {
  const int n_qtiles = (int)(((uint64_t)(a.Hq / a.Hkv) * a.N + kBr - 1) / kBr);
  const uint64_t grid = (uint64_t)n_qtiles * a.Hkv * a.B;
  const float c_log2 = a.scale * 1.44269504088896341f;
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, kNeg>), dim3((uint32_t)grid), dim3(kThreads), 0,
                     a.stream, static_cast<const uint8_t*>(a.q), static_cast<const uint8_t*>(a.k),
                     static_cast<const uint8_t*>(a.v), static_cast<__bf16*>(a.o), a.lse, a.Hq,
                     a.Hkv, a.N, fp8_padded_keys(a.N), c_log2, a.v_scale, n_qtiles,
                     (uint32_t)a.n_xcd);
  return hipGetLastError();
}

}  // namespace

int fp8_padded_keys(int N) { return (N + 15) / 16 * 16; }

uint64_t fwd_fp8_grid(int B, int Hq, int Hkv, int N) {
  return ((uint64_t)(Hq / Hkv) * N + kBr - 1) / kBr * Hkv * B;
}

hipError_t launch_fwd_fp8(const FwdArgs& a) {
  const bool neg = a.scale < 0.0f;
  if (a.d == 128) return neg ? launch_d<128, true>(a) : launch_d<128, false>(a);
  return neg ? launch_d<64, true>(a) : launch_d<64, false>(a);
}

}  // namespace attn
