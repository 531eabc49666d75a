// attn_fwd_bf16_rows32.hip -- fused, tiled attention forward for gfx950,
// bf16 I/O, one 32-row query block per wave (head dim 64; head dim 128 where
// the keys are short or the grid is small, as chosen in kernels.hpp).
//
// The IO-aware forward (blog "attention 的显存线性化", section 三; the
// "efficient attention" chapter's online-softmax paragraph): one workgroup
// owns kBr query rows of one head and streams every key/value tile of that
// head through LDS, keeping per row a running maximum m and exp-sum l and
// an fp32 output accumulator.  S and P only ever exist in registers.
//
// Design for CDNA4:
//  * 4 waves x 32 query rows; at head dim 64 the kernel fits 128 VGPRs and
//    32 KB of LDS, so four workgroups (four waves per SIMD) share a CU: at
//    d = 64 the softmax has as many vector instructions per MFMA as at
//    d = 128 has per two, and the other waves' instructions fill the gaps
//    one wave leaves while it waits on its own dependencies.  At head dim
//    128 (214 VGPRs, 64 KB of LDS) two workgroups share a CU.
//  * Each wave computes S^T = K Q^T per 32-key
//    block with v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, the
//    wave's Q rows resident in VGPRs as the B operand).  In that output
//    layout a lane owns ONE query (column l % 32) and 16 of the 32 keys, so
//    the row max / row sum are in-lane reductions plus one v_permlane32_swap
//    with the other half-wave.
//  * O^T = V^T P^T on the same MFMA: P^T comes straight from the S^T
//    accumulator registers (rounded to bf16); the V^T operand is read from
//    the row-major V tile with ds_read_b64_tr_b16, which hands each lane
//    four consecutive keys of one d column.  The O^T accumulator again gives
//    each lane one query, so the rescale by exp(m_old - m_new) is a per-lane
//    scalar.
//  * K and V tiles (64 keys) go global -> LDS directly (buffer_load ... lds,
//    no staging registers), two stages, the next tile in flight while the
//    current one is computed.  Rows sit unpadded with their 16-byte chunks
//    XOR-swizzled by the row index, so both the MFMA operand reads of K and
//    the transposing reads of V are free of LDS bank conflicts.
//  * The scale is folded into exp2: p = 2^(s * scale * log2 e - m).  Since
//    softmax is unchanged by any common shift of a row (the basis of the
//    rescale rule), m need only keep the weights bounded: a full tile is
//    weighted against m as it stands and kept if its exp-sum stays under a
//    cap; only the first tile, the tail tile and a tile over the cap take
//    the tile's row max, move m and rescale the accumulator.
//  * Workgroups of one K/V head are numbered consecutively and remapped so
//    they run on one XCD and share its L2.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kFWaves = 4;
constexpr int kFThreads = kFWaves * kWave;
constexpr int kFRows = 32;                   // query rows per wave
constexpr int kFBr = kFWaves * kFRows;       // query rows per workgroup
constexpr float kSumCap = 65536.0f;          // largest per-lane exp-sum of a tile kept as is

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int D>
struct FGeo {
  static constexpr int kBc = 64;                      // keys per tile
  static constexpr int kKB = kBc / 32;                 // 32-key blocks per tile
  static constexpr int kKSteps = D / 16;               // MFMA k-steps over d
  static constexpr int kDB = D / 32;                   // 32-wide d blocks
  static constexpr int kCPR = D / 8;                   // 16-byte chunks per row
  static constexpr int kTile = kBc * D;                // bf16 elements of K (or V)
  static constexpr int kStage = 2 * kTile;             // K then V
  static constexpr int kDmaPerWave = kTile / 8 / kWave / kFWaves;   // 16-B loads per lane per tile
  static_assert(kDmaPerWave * 8 * kWave * kFWaves == kTile, "tile must split over the waves");
};

// Chunk swizzle: chunk c of row r is stored at chunk c ^ swz<D>(r), which
// keeps both read patterns free of LDS bank conflicts on gfx950 (64 banks,
// 256 bytes per cycle; measured: 4.7 cycles per ds_read_b128 of K and
// 3.1 - 4.2 per transposing read of V, against 8.4 - 8.6 with a 3-bit swizzle):
//  * K operand reads: lanes 0..15 read one chunk of rows r..r+15 (r % 16 ==
//    0); the 16 (d = 128, 256-byte rows) or 2 x 8 (d = 64, two 128-byte rows
//    per bank cycle) chunks must land on distinct banks;
//  * transposing V reads: four rows x four 8-byte columns per 16 lanes.
// d = 128: bits (r1 r0 r2 r3) of the row; d = 64: bits (r1 r2 r3).
template <int D>
__device__ __forceinline__ int swz(int row) {
  return D == 128 ? (((row & 3) << 1) | ((row >> 2) & 1) | (row & 8))
                  : ((((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1));
}

// clamp(rem, 0, hi) on the scalar unit.  Written as scalar instructions so
// the count never takes a detour through a vector register (v_med3 and
// v_readfirstlane), which would tie the tile loads to the vector pipeline.
__device__ __forceinline__ int srows(int rem, int hi) {
  int r;
  asm("s_max_i32 %0, %1, 0\n\ts_min_i32 %0, %0, %2" : "=&s"(r) : "s"(rem), "s"(hi) : "scc");
  return r;
}

// Issue the direct loads of one K or V tile (keys j0 .. j0 + kBc - 1) into
// the LDS tile at byte address lds_tile.  The buffer covers only rows
// j0 .. N-1: rows past N read as zeros (the softmax masks them) and nothing
// is read out of bounds.  Issued as inline assembly so the compiler does not
// see an LDS write in flight and does not hold the reads of the other buffer
// behind it; wait_dma() and the barrier order these loads against readers.
template <int D>
__device__ __forceinline__ void dma_tile(const __bf16* __restrict__ head, int j0, int N,
                                         uint32_t lds_tile, int wave, const int* dvoff) {
  using G = FGeo<D>;
  const int rows = srows(N - j0, G::kBc);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(head) + (int64_t)min(j0, N) * D, (short)0, rows * D * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < G::kDmaPerWave; ++i) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(
        lds_tile + (uint32_t)((wave * G::kDmaPerWave + i) * kWave * 16));
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 ::"s"(dst), "v"(dvoff[i]), "s"(rs) : "memory");
  }
}

// s_waitcnt vmcnt(0) as a real instruction (expcnt and lgkmcnt left at
// their maxima), so the compiler knows every vector load has completed.
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// IEEE-754 maximum / minimum (v_maximum3_f32 / v_minimum3_f32 on gfx950):
// unlike fmaxf they need no canonicalisation of MFMA results first.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmin(float a, float b) { return __builtin_elementwise_minimum(a, b); }

// Across the two half-waves (lane l and l ^ 32): both get the combined value.
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

// This lane's part of the exp-sum of one tile (its 16 keys per 32-key
// block), in fp32: four independent chains, then their sum.
template <int KB>
__device__ __forceinline__ float lane_sum(const float (&p)[KB][16]) {
  float ps[4] = {p[0][0], p[0][1], p[0][2], p[0][3]};
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int e = (kb == 0 ? 4 : 0); e < 16; ++e) ps[e & 3] += p[kb][e];
  return (ps[0] + ps[1]) + (ps[2] + ps[3]);
}

template <int D, bool kNegScale>
__global__ __launch_bounds__(kFThreads, D == 64 ? 4 : 2)
void attn_fwd_bf16_rows32_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                          const __bf16* __restrict__ v, __bf16* __restrict__ o,
                          float* __restrict__ lse, int Hq, int Hkv, int N, float c_log2,
                          int n_qtiles, uint32_t n_xcd) {
  using G = FGeo<D>;
  __shared__ __align__(16) __bf16 smem[2 * G::kStage];

  const uint32_t lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) __bf16*)smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // direct loads: instruction i of this wave fills 16-byte chunks
  // slot .. slot + 63 of a tile; lane's chunk g = slot + lane holds logical
  // chunk (g % kCPR) ^ swz<D>(row) of row g / kCPR
  int dvoff[G::kDmaPerWave];
#pragma unroll
  for (int i = 0; i < G::kDmaPerWave; ++i) {
    const int g = (wave * G::kDmaPerWave + i) * kWave + lane;
    const int row = g / G::kCPR;
    const int c = (g % G::kCPR) ^ swz<D>(row);
    dvoff[i] = (row * D + c * 8) * 2;
  }

  // ---- which (b, K/V head, query tile) this workgroup owns ----------------
  // The query heads that share a K/V head are adjacent in q, o and lse, so
  // the rows of a group form one block of (Hq / Hkv) * N rows; query tiles
  // run over that block (a tile may end in one head and go on in the next),
  // so one K/V stream serves every head of the group and heads shorter than
  // a tile leave no rows idle.  Query tiles are numbered fastest: workgroups
  // that stream the same K/V rows at the same time run side by side on one
  // XCD and share its L2.
  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x, n_xcd);
  const int qt = (int)(logical % (uint32_t)n_qtiles);
  const uint32_t rest = logical / (uint32_t)n_qtiles;
  const int kvh = (int)(rest % (uint32_t)Hkv);
  const int b = (int)(rest / (uint32_t)Hkv);

  const int n_qrows = (Hq / Hkv) * N;                                // rows of the group
  const int64_t head_q = ((int64_t)b * Hkv + kvh) * (int64_t)n_qrows; // its first row
  const int64_t head_kv = ((int64_t)b * Hkv + kvh) * (int64_t)N;
  const __bf16* kh = k + head_kv * D;
  const __bf16* vh = v + head_kv * D;

  const int n_tiles = (N + G::kBc - 1) / G::kBc;
  // first tile in flight before anything else
  dma_tile<D>(kh, 0, N, lds, wave, dvoff);
  dma_tile<D>(vh, 0, N, lds + G::kTile * 2, wave, dvoff);

  const int qrow = qt * kFBr + wave * kFRows + l32;   // this lane's query
  const bool qvalid = qrow < n_qrows;

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

  // ---- per-lane LDS offsets (elements) -------------------------------------
  // K operand: row kb*32 + l32, chunk 2 s + hh, swizzled by the row.
  int koff[G::kKSteps];
#pragma unroll
  for (int s = 0; s < G::kKSteps; ++s) koff[s] = l32 * D + (((2 * s + hh) ^ swz<D>(l32)) * 8);
  // V^T operand (transposing read): in each 16-lane group, lane i points at
  // key (i / 4) of a 4-key run and d columns 4 (i % 4) .. +3 of the group's
  // 16 columns; it receives key run 0..3 of column (group base + i).
  const int li = lane & 15;
  const int dhalf = (lane >> 4) & 1;
  const int vrow = 4 * hh + (li >> 2);          // row within a 16-key step (plus 8 for slots 4..7)
  int voff[G::kDB], voff8[G::kDB];
#pragma unroll
  for (int db = 0; db < G::kDB; ++db) {
    const int dcol = db * 32 + dhalf * 16 + 4 * (li & 3);
    voff[db] = vrow * D + (((dcol >> 3) ^ swz<D>(vrow)) * 8) + (dcol & 7);
    voff8[db] = (vrow + 8) * D + (((dcol >> 3) ^ swz<D>(vrow + 8)) * 8) + (dcol & 7);
  }

  f32x16 oacc[G::kDB];
#pragma unroll
  for (int i = 0; i < G::kDB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;   // running max of the log2-scaled scores
  float l_run = 0.0f;        // this lane's part of the exp-sum (its 16 keys per block)

  wait_dma();
  __syncthreads();

  // One key tile in LDS stage `stage` (a compile-time constant: the loop
  // below runs two tiles per trip, so every LDS read has a fixed offset).
  auto tile = [&](const int jt, auto stage_c) {
    constexpr int stage = decltype(stage_c)::value;
    const __bf16* ks = smem + stage * G::kStage;
    const __bf16* vs = ks + G::kTile;
    if (jt + 1 < n_tiles) {
      const uint32_t nxt = lds + (1 - stage) * G::kStage * 2;
      dma_tile<D>(kh, (jt + 1) * G::kBc, N, nxt, wave, dvoff);
      dma_tile<D>(vh, (jt + 1) * G::kBc, N, nxt + G::kTile * 2, wave, dvoff);
    }

    // ---- S^T = K Q^T for kKB blocks of 32 keys ---------------------------
    auto scores = [&](f32x16 (&sa)[G::kKB], const __bf16* kt) {
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb) {
        bf16x8 kf[G::kKSteps];
#pragma unroll
        for (int s = 0; s < G::kKSteps; ++s)
          kf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + kb * 32 * D + koff[s]));
        sa[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < G::kKSteps; ++s) sa[kb] = mfma32x32x16(kf[s], qf[s], sa[kb]);
      }
    };
    // ---- online softmax on this lane's 16 * kKB scores -------------------
    // Fast path (every full tile after the first): weights against the
    // running max as it stands, p = 2^(s c - m), with no max over the tile.
    // m only has to bound the weights, not equal the row max (any common
    // shift of a row leaves its softmax unchanged), so the tile is kept as
    // long as the lane's exp-sum over it stays <= kSumCap; that also bounds
    // every weight.  Otherwise (first tile, tail tile, a sum above the cap,
    // or not finite) the full step takes the tile's row max, moves m and
    // rescales the accumulators first; it computes the scores itself, from
    // the K tile still in LDS, so that the fast path need not keep its
    // scores beside the weights for a tile that fails the cap.
    const int j0 = jt * G::kBc;
    const bool tail = j0 + G::kBc > N;
    float p[G::kKB][16];
    float tsum;
    bool redo = tail || jt == 0;
    if (!redo) {
      f32x16 sacc[G::kKB];
      scores(sacc, ks);
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) p[kb][e] = exp2_fast(__builtin_fmaf(sacc[kb][e], c_log2, -m_run));
      tsum = lane_sum<G::kKB>(p);
      redo = __any(!(tsum <= kSumCap));
    }
    if (redo) {
      // the tile's offset goes through an empty asm statement so that the
      // compiler cannot merge these reads and products with the ones above
      int off = stage * G::kStage;
      asm volatile("" : "+s"(off));
      f32x16 sre[G::kKB];
      scores(sre, smem + off);
      float ext;
      if (!tail) {
        // tree of max (min) over the lane's scores
        float t[G::kKB * 4];
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const f32x16& a = sre[kb];
            t[kb * 4 + r] = kNegScale
                ? vmin(vmin(a[4 * r], a[4 * r + 1]), vmin(a[4 * r + 2], a[4 * r + 3]))
                : vmax(vmax(a[4 * r], a[4 * r + 1]), vmax(a[4 * r + 2], a[4 * r + 3]));
          }
#pragma unroll
        for (int w = G::kKB * 4; w > 1; w >>= 1)
#pragma unroll
          for (int i = 0; i < w / 2; ++i)
            t[i] = kNegScale ? vmin(t[i], t[i + w / 2]) : vmax(t[i], t[i + w / 2]);
        ext = kNegScale ? xhalf_min(t[0]) : xhalf_max(t[0]);
      } else {
        // keys >= N (zero rows) are not part of the softmax: leave them out
        float e2 = kNegScale ? INFINITY : -INFINITY;
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = j0 + kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
            if (key < N) e2 = kNegScale ? vmin(e2, sre[kb][e]) : vmax(e2, sre[kb][e]);
          }
        ext = kNegScale ? xhalf_min(e2) : xhalf_max(e2);
      }
      ext *= c_log2;   // the row's max of s * c_log2

      // m moves up to the row max seen so far (never down); the rescale
      // factor is 1 for rows whose max did not grow.  On the first tile
      // there is nothing to rescale yet (O and l are zero).
      if (jt == 0) {
        m_run = ext;
      } else if (__any(ext > m_run)) {
        const float m_new = fmaxf(m_run, ext);
        const float alpha = exp2_fast(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < G::kDB; ++i) oacc[i] *= alpha;
      }

#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) p[kb][e] = exp2_fast(__builtin_fmaf(sre[kb][e], c_log2, -m_run));
      if (tail) {
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = j0 + kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
            if (key >= N) p[kb][e] = 0.0f;
          }
      }
      tsum = lane_sum<G::kKB>(p);
    }
    l_run += tsum;

    // ---- O^T += V^T P^T ---------------------------------------------------
    // P^T slot (hh, e) of k-step s2 in block kb holds key
    // kb*32 + 16 s2 + 8 (e / 4) + 4 hh + e % 4; the transposing V reads
    // fetch the same keys: slots 0..3 from rows +0..3, slots 4..7 from +8..11.
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 pu;
#pragma unroll
        for (int w = 0; w < 4; ++w) pu[w] = pack_bf16x2(p[kb][8 * s2 + 2 * w], p[kb][8 * s2 + 2 * w + 1]);
        const bf16x8 pf = as_bf16x8(pu);
        const int rbase = (kb * 32 + 16 * s2) * D;
#pragma unroll
        for (int db = 0; db < G::kDB; ++db) {
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vs + rbase + voff[db]));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vs + rbase + voff8[db]));
          const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, a8), pf, oacc[db]);
        }
      }

    wait_dma();
    __syncthreads();
  };
  for (int jt = 0; jt < n_tiles; jt += 2) {
    tile(jt, std::integral_constant<int, 0>{});
    if (jt + 1 < n_tiles) tile(jt + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: O = O~ / l, lse = (m + log2 l) ln 2 ------------------------
  const float l_tot = xhalf_sum(l_run);
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
  const int n_qtiles = (int)(((uint64_t)(a.Hq / a.Hkv) * a.N + kFBr - 1) / kFBr);
  const uint64_t grid = (uint64_t)n_qtiles * a.Hkv * a.B;
  const float c_log2 = a.scale * 1.44269504088896341f;
  hipLaunchKernelGGL((attn_fwd_bf16_rows32_kernel<D, kNeg>), dim3((uint32_t)grid), dim3(kFThreads), 0,
                     a.stream, static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<__bf16*>(a.o), a.lse, a.Hq,
                     a.Hkv, a.N, c_log2, n_qtiles, (uint32_t)a.n_xcd);
  return hipGetLastError();
}

}  // namespace

uint64_t fwd_bf16_rows32_grid(int B, int Hq, int Hkv, int N) {
  return ((uint64_t)(Hq / Hkv) * N + kFBr - 1) / kFBr * Hkv * B;
}

hipError_t launch_fwd_bf16_rows32(const FwdArgs& a) {
  if (a.d == 128) return a.scale < 0.0f ? launch_d<128, true>(a) : launch_d<128, false>(a);
  if (a.d != 64) return hipErrorInvalidValue;
  return a.scale < 0.0f ? launch_d<64, true>(a) : launch_d<64, false>(a);
}

}  // namespace attn
