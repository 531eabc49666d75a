// attn_bwd.hip -- attention backward for gfx950: dQ, dK, dV from Q, K, V, O,
// dO and the forward's lse, bf16 I/O, fp32 accumulation.
//
// The pages' backward (blog "attention 的显存线性化", section 五; the
// "efficient attention" chapter's online-softmax section): the [N, N]
// matrices of the forward are not kept; each block of S and P is recomputed
// from Q, K and the saved per-row statistics when it is needed.  With the
// forward's lse, P = exp(scale * Q K^T - lse) exactly, with no running max.
// For the loss gradient dO = dL/dO the gradients of O = P V, P = softmax(S)
// are (the chain rule through a row softmax):
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),  D_i = sum_c dO_ic O_ic,
//   dQ = scale * dS K,   dK = scale * dS^T Q
// (D_i = sum_j P_ij dP_ij, the row sum the softmax Jacobian subtracts).
//
// Two kernels, in this order:
//   attn_bwd_dq      -- one workgroup per 256 query rows: the K / V tiles of
//                       the head stream through LDS (as in the forward) and dQ
//                       accumulates in registers; each row's D_i (fp32, from
//                       the dO rows it holds and O) goes to the caller's
//                       workspace;
//   attn_bwd_dkdv    -- one workgroup per 128 keys of a K/V head (head dim
//                       64; attn_bwd_dkdv_w64 at 128: 256 keys, 64 per
//                       wave): the keys' K and V rows stay in registers while
//                       the Q / dO tiles (and lse, D) of every query head of
//                       the group stream through LDS; dK and dV accumulate in
//                       registers and are written once; no atomics anywhere.
// S and dP are computed twice (once per kernel): 7 products per (query, key)
// block instead of 5, traded for no atomic adds and no [N, N] storage.
//
// Layouts (v_mfma_f32_32x32x16_bf16; see mfma32x32x16 for operand slots):
//  * dkdv: S = Q K^T and dP = dO V^T with the wave's K / V rows as the B
//    operand (lane = key), so a lane holds 16 queries of one key; P and dS
//    packed to bf16 are then directly the B operand of dV^T = dO^T P and
//    dK^T = Q^T dS, whose A operands (dO^T, Q^T) come from transposing LDS
//    reads of the row-major tiles.
//  * dq: S^T = K Q^T and dP^T = V dO^T with the wave's Q / dO rows as the B
//    operand (lane = query: lse and D are per-lane scalars); dS^T packed is
//    the B operand of dQ^T = K^T dS^T, K^T read transposed from LDS.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kBWaves = 4;
constexpr int kBThreads = kBWaves * kWave;
constexpr int kWRows = 32;                    // rows a wave owns (keys in dkdv, queries in dq)
constexpr int kWgRows = kBWaves * kWRows;     // rows a workgroup owns
constexpr int kTRows = 64;                    // rows of a streamed LDS tile
constexpr float kLog2e = 1.44269504088896341f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

template <int D, int R = kTRows>
struct BGeo {
  static constexpr int kKSteps = D / 16;               // MFMA k-steps over d
  static constexpr int kDB = D / 32;                   // 32-wide d blocks
  static constexpr int kCPR = D / 8;                   // 16-byte chunks per row
  static constexpr int kTile = R * D;                  // bf16 elements of one R-row tile
  static constexpr int kDma = kTile / 8 / kBThreads;   // 16-byte loads per lane per tile
  static_assert(kDma * 8 * kBThreads == kTile, "tile must split over the workgroup");
};

// Chunk c of row r of a tile sits at chunk c ^ swz(r): both the 16-byte row
// reads (MFMA A operands) and the transposing 8-byte reads are free of LDS
// bank conflicts (the forward kernels' layout).
template <int D>
__device__ __forceinline__ int swz(int row) {
  return D == 128 ? (((row & 3) << 1) | ((row >> 2) & 1) | (row & 8))
                  : ((((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1));
}

__device__ __forceinline__ int srows(int rem, int hi) {
  int r;
  asm("s_max_i32 %0, %1, 0\n\ts_min_i32 %0, %0, %2" : "=&s"(r) : "s"(rem), "s"(hi) : "scc");
  return r;
}

// Rows j0 .. j0 + R - 1 of a [N, D] bf16 array -> the LDS tile at byte
// address lds_tile, global -> LDS directly.  The buffer covers only rows
// j0 .. N-1: rows past N read as zeros and nothing is read out of bounds.
// Inline assembly, as in the forward: the waits below order it against
// readers.
template <int D, int R = kTRows>
__device__ __forceinline__ void dma_tile(const __bf16* __restrict__ base, int j0, int N,
                                         uint32_t lds_tile, int wave, const int* dvoff) {
  using G = BGeo<D, R>;
  const int rows = srows(N - j0, R);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(base) + (int64_t)min(j0, N) * D, (short)0, rows * D * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < G::kDma; ++i) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(
        lds_tile + (uint32_t)((wave * G::kDma + i) * kWave * 16));
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 ::"s"(dst), "v"(dvoff[i]), "s"(rs) : "memory");
  }
}

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Per-lane LDS byte offsets of one tile's operand reads.
template <int D, int R = kTRows>
struct TileOffsets {
  int dvoff[BGeo<D, R>::kDma];  // this lane's 16-byte chunks of a tile load
  int row[BGeo<D>::kKSteps];    // 16-byte row read: row l32, chunk 2 s + hh
  int tr[BGeo<D>::kDB];         // transposing read, rows +0..3 of a 16-row step
  int tr8[BGeo<D>::kDB];        // the same, rows +8..11
};

template <int D, int R = kTRows>
__device__ __forceinline__ TileOffsets<D, R> tile_offsets(int lane, int wave) {
  using G = BGeo<D, R>;
  TileOffsets<D, R> t;
  const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int i = 0; i < G::kDma; ++i) {
    const int g = (wave * G::kDma + i) * kWave + lane;
    const int row = g / G::kCPR;
    t.dvoff[i] = (row * D + (((g % G::kCPR) ^ swz<D>(row)) * 8)) * 2;
  }
#pragma unroll
  for (int s = 0; s < G::kKSteps; ++s) t.row[s] = (l32 * D + (((2 * s + hh) ^ swz<D>(l32)) * 8)) * 2;
  // transposing read: in each 16-lane group, lane i points at row (i / 4)
  // of a 4-row run and columns 4 (i % 4) .. +3 of the group's 16 columns;
  // it receives rows 0..3 of column (group base + i)
  const int li = lane & 15, dhalf = (lane >> 4) & 1;
  const int vrow = 4 * hh + (li >> 2);
#pragma unroll
  for (int db = 0; db < G::kDB; ++db) {
    const int dcol = db * 32 + dhalf * 16 + 4 * (li & 3);
    t.tr[db] = (vrow * D + (((dcol >> 3) ^ swz<D>(vrow)) * 8) + (dcol & 7)) * 2;
    t.tr8[db] = ((vrow + 8) * D + (((dcol >> 3) ^ swz<D>(vrow + 8)) * 8) + (dcol & 7)) * 2;
  }
  return t;
}

// A operand, rows r0 + l32 of the tile at byte address tile, k-step s.
__device__ __forceinline__ bf16x8 lds_row(uint32_t tile, int off) {
  const u32x4 u = *(const lds_u32x4*)(uintptr_t)(tile + off);
  return as_bf16x8(u);
}

// A operand of a transposed product: columns = tile rows (16-row k-step at
// byte offset rbase), rows = d block db.  Slot (hh, j) holds tile row
// 8 (j / 4) + 4 hh + j % 4 of the step, matching the accumulator layout the
// B operand comes from.
__device__ __forceinline__ bf16x8 lds_tr(uint32_t tile, int off, int off8) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(tile + off));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(tile + off8));
  const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, a8);
}

// B operand from global memory: d = 16 s + 8 hh .. +7 of row `row` (rows
// past N read row N - 1; their results are never used).
template <int D>
__device__ __forceinline__ void load_rowfrags(bf16x8 (&f)[BGeo<D>::kKSteps],
                                              const __bf16* __restrict__ base, int row, int N,
                                              int hh) {
  const __bf16* p = base + (int64_t)min(row, N - 1) * D + 8 * hh;
#pragma unroll
  for (int s = 0; s < BGeo<D>::kKSteps; ++s) f[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(p + 16 * s));
}

// Store the transposed accumulator of a wave (rows = d, column = this
// lane's row `row`), times `mul`, as bf16 row `row` of out.
template <int D>
__device__ __forceinline__ void store_rowT(const f32x16 (&acc)[BGeo<D>::kDB], __bf16* __restrict__ out,
                                           float mul, int hh) {
#pragma unroll
  for (int db = 0; db < BGeo<D>::kDB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      u32x2 w;
      w[0] = pack_bf16x2(acc[db][4 * r + 0] * mul, acc[db][4 * r + 1] * mul);
      w[1] = pack_bf16x2(acc[db][4 * r + 2] * mul, acc[db][4 * r + 3] * mul);
      *reinterpret_cast<u32x2*>(out + db * 32 + 8 * r + 4 * hh) = w;
    }
}

// ---------------------------------------------------------------------------
// dK, dV at head dim 64: one workgroup per 128 keys of K/V head (b, kvh),
// two workgroups (two waves per SIMD) per CU; each wave owns 32 keys and
// runs all four products for them.
template <int D>
__global__ __launch_bounds__(kBThreads, 2)
void attn_bwd_dkdv_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                          const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
                          const float* __restrict__ lse, const float* __restrict__ dvec,
                          __bf16* __restrict__ dk, __bf16* __restrict__ dv, int Hq, int Hkv,
                          int N, float c_log2, float scale, int n_ktiles, uint32_t n_xcd) {
  using G = BGeo<D>;
  // per stage: Q tile, dO tile (bf16), then lse*log2e and D of its 64 rows
  constexpr uint32_t kTileB = G::kTile * 2;
  constexpr uint32_t kStageB = 2 * kTileB + 2 * kTRows * 4;
  __shared__ __align__(16) unsigned char smem[2 * kStageB];
  const uint32_t lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // key tiles fastest: the workgroups of one K/V head stream the same Q/dO
  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x, n_xcd);
  const int kt = (int)(logical % (uint32_t)n_ktiles);
  const uint32_t rest = logical / (uint32_t)n_ktiles;
  const int kvh = (int)(rest % (uint32_t)Hkv);
  const int b = (int)(rest / (uint32_t)Hkv);
  const int64_t head_kv = ((int64_t)b * Hkv + kvh) * (int64_t)N;
  // the query heads of the group are adjacent in q, dO, lse and D: their
  // rows form one block of (Hq / Hkv) * N rows, streamed 64 at a time
  const int n_qrows = (Hq / Hkv) * N;
  const int64_t head_q = ((int64_t)b * Hkv + kvh) * (int64_t)n_qrows;

  const int krow = kt * kWgRows + wave * kWRows + l32;   // this lane's key (B operand column)
  static_assert(D == 64, "head dim 128 runs attn_bwd_dkdv_w64_kernel");
  bf16x8 kf[G::kKSteps], vf[G::kKSteps];
  load_rowfrags<D>(kf, k + head_kv * D, krow, N, hh);
  load_rowfrags<D>(vf, v + head_kv * D, krow, N, hh);

  const TileOffsets<D> off = tile_offsets<D>(lane, wave);
  f32x16 dkacc[G::kDB], dvacc[G::kDB];
#pragma unroll
  for (int i = 0; i < G::kDB; ++i) {
    dkacc[i] = f32x16{};
    dvacc[i] = f32x16{};
  }

  const int n_steps = (n_qrows + kTRows - 1) / kTRows;   // 64-row query tiles of the group

  // Loads of step t into stage t & 1: the Q and dO tiles go global -> LDS
  // directly; lse and D of the 64 rows come through registers (rows past
  // the group's last get lse = +inf, so their weights are exp2(-inf) = 0,
  // and D = 0).  The row statistics are loaded before the tiles and scaled
  // only when committed: a use right after the load would make the wave
  // wait for every load in flight, the tile loads issued just before
  // included (the wait counter counts them all, in order).
  float st_lse = 0.0f, st_d = 0.0f;
  auto issue = [&](int t) {
    const int q0 = t * kTRows;
    const uint32_t stage = lds + (uint32_t)(t & 1) * kStageB;
    if (tid < kTRows) {
      const int row = q0 + tid;
      st_lse = row < n_qrows ? lse[head_q + row] : INFINITY;
      st_d = row < n_qrows ? dvec[head_q + row] : 0.0f;
    }
    dma_tile<D>(q + head_q * D, q0, n_qrows, stage, wave, off.dvoff);
    dma_tile<D>(dout + head_q * D, q0, n_qrows, stage + kTileB, wave, off.dvoff);
  };
  auto commit = [&](int t) {   // after the loads of step t have landed
    if (tid < kTRows) {
      const uint32_t stage = lds + (uint32_t)(t & 1) * kStageB;
      *(__attribute__((address_space(3))) float*)(uintptr_t)(stage + 2 * kTileB + tid * 4) = st_lse * kLog2e;
      *(__attribute__((address_space(3))) float*)(uintptr_t)(stage + 2 * kTileB + kTRows * 4 + tid * 4) = st_d;
    }
  };

  issue(0);
  wait_vm();
  commit(0);
  __syncthreads();

  // one query step in LDS stage `st` (a compile-time constant: the loop
  // below runs two steps per trip, so every LDS read has a fixed offset)
  auto q_step = [&](const int t, auto stage_c) {
    constexpr int st = decltype(stage_c)::value;
    const uint32_t stage = lds + (uint32_t)st * kStageB;
    const uint32_t qtile = stage, dotile = stage + kTileB;
    const uint32_t lse_s = stage + 2 * kTileB, d_s = lse_s + kTRows * 4;
    if (t + 1 < n_steps) issue(t + 1);

    // block by block (two waves per SIMD: the other wave fills in)
#pragma unroll
    for (int qb = 0; qb < kTRows / 32; ++qb) {
      // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int s = 0; s < G::kKSteps; ++s) {
        const bf16x8 qa = lds_row(qtile + qb * 32 * D * 2, off.row[s]);
        const bf16x8 da = lds_row(dotile + qb * 32 * D * 2, off.row[s]);
        sacc = mfma32x32x16(qa, kf[s], sacc);
        pacc = mfma32x32x16(da, vf[s], pacc);
      }
      // element 4 r + j: query qb*32 + 8 r + 4 hh + j
      float p[16], ds[16];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 l4 = *(const lds_f32x4*)(uintptr_t)(lse_s + (qb * 32 + 8 * r + 4 * hh) * 4);
        const f32x4 d4 = *(const lds_f32x4*)(uintptr_t)(d_s + (qb * 32 + 8 * r + 4 * hh) * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * r + j;
          p[e] = exp2_fast(__builtin_fmaf(sacc[e], c_log2, -l4[j]));
          ds[e] = p[e] * (pacc[e] - d4[j]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the two 16-query k-steps
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 pu, du;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pu[w] = pack_bf16x2(p[8 * s2 + 2 * w], p[8 * s2 + 2 * w + 1]);
          du[w] = pack_bf16x2(ds[8 * s2 + 2 * w], ds[8 * s2 + 2 * w + 1]);
        }
        const uint32_t rb = (uint32_t)((qb * 32 + 16 * s2) * D * 2);
#pragma unroll
        for (int db = 0; db < G::kDB; ++db) {
          dvacc[db] = mfma32x32x16(lds_tr(dotile + rb, off.tr[db], off.tr8[db]), as_bf16x8(pu), dvacc[db]);
          dkacc[db] = mfma32x32x16(lds_tr(qtile + rb, off.tr[db], off.tr8[db]), as_bf16x8(du), dkacc[db]);
        }
      }
    }
    wait_vm();
    if (t + 1 < n_steps) commit(t + 1);
    __syncthreads();
  };
  for (int t = 0; t < n_steps; t += 2) {
    q_step(t, std::integral_constant<int, 0>{});
    if (t + 1 < n_steps) q_step(t + 1, std::integral_constant<int, 1>{});
  }

  if (krow < N) {
    store_rowT<D>(dkacc, dk + (head_kv + krow) * D, scale, hh);
    store_rowT<D>(dvacc, dv + (head_kv + krow) * D, 1.0f, hh);
  }
}

// ---------------------------------------------------------------------------
// acc += a b on the matrix core with the accumulator in AGPRs (the d = 128
// dK/dV kernel below needs both register files: dK and dV fill the AGPRs,
// everything else uses VGPRs; the compiler places all accumulators of a
// kernel in one file).  A matrix-core read of a register the vector ALU
// wrote needs two wait states in between: kNop when b may have been
// written within the last two instructions.  Back-to-back products into
// the same accumulator need none.
template <bool kNop>
__device__ __forceinline__ void mfma_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (kNop)
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// acc = a b, the first product of a chain (the accumulator starts in AGPRs).
template <bool kNop>
__device__ __forceinline__ void mfma_agpr_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (kNop)
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}

// dK and dV at head dim 128 (written for 64 and 128; launched at 128): one
// workgroup of four waves (one per SIMD) per 256 keys of K/V head (b, kvh);
// each wave owns 64 keys (two 32-key blocks) and runs all four products for
// them: S = Q K^T, dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS.  K
// and V of its keys stay in VGPRs (128 at d = 128), dK and dV in AGPRs
// (256); every Q / dO operand read from LDS feeds one product per key
// block, and P stays in registers.  A step covers 32 query rows; the next
// tile loads during the step (two LDS slots).
constexpr int kW64Keys = 64;                    // keys a wave owns
constexpr int kW64Rows = 32;                    // query rows per step
constexpr int kW64WgKeys = kBWaves * kW64Keys;  // keys a workgroup owns

template <int D>
__global__ __launch_bounds__(kBThreads, 1)
void attn_bwd_dkdv_w64_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                              const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
                              const float* __restrict__ lse, const float* __restrict__ dvec,
                              __bf16* __restrict__ dk, __bf16* __restrict__ dv, int Hq, int Hkv,
                              int N, float c_log2, float scale, int n_ktiles, uint32_t n_xcd) {
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  using G = BGeo<D, kW64Rows>;
  constexpr int kKB = kW64Keys / 32;                         // 32-key blocks per wave
  constexpr int kNS = 2 * G::kKSteps;                        // vector slots of phases 2 and 3
  constexpr int kEPS = 32 / kNS;                             // values per slot: 2 (d = 128), 4
  static_assert(kNS == 4 * G::kDB && kEPS % 2 == 0, "slot layout");
  constexpr uint32_t kTileB = G::kTile * 2;
  constexpr uint32_t kStatB = 2 * kW64Rows * 4;              // lse and D of one tile
  constexpr uint32_t kStageB = 2 * kTileB + kStatB;          // Q, dO, lse, D
  constexpr uint32_t kOutB = kW64Keys * D * 2;               // one wave's dK or dV, bf16
  constexpr uint32_t kSmem = 2 * kStageB > kBWaves * kOutB ? 2 * kStageB : kBWaves * kOutB;
  __shared__ __align__(16) unsigned char smem[kSmem];
  const uint32_t lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x, n_xcd);
  const int kt = (int)(logical % (uint32_t)n_ktiles);
  const uint32_t rest = logical / (uint32_t)n_ktiles;
  const int kvh = (int)(rest % (uint32_t)Hkv);
  const int b = (int)(rest / (uint32_t)Hkv);
  const int64_t head_kv = ((int64_t)b * Hkv + kvh) * (int64_t)N;
  const int n_qrows = (Hq / Hkv) * N;
  const int64_t head_q = ((int64_t)b * Hkv + kvh) * (int64_t)n_qrows;

  const int krow0 = kt * kW64WgKeys + wave * kW64Keys + l32;   // this lane's key in block 0
  bf16x8 kf[kKB][G::kKSteps], vf[kKB][G::kKSteps];
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb) {
    load_rowfrags<D>(kf[kb], k + head_kv * D, krow0 + 32 * kb, N, hh);
    load_rowfrags<D>(vf[kb], v + head_kv * D, krow0 + 32 * kb, N, hh);
  }

  const TileOffsets<D, kW64Rows> off = tile_offsets<D, kW64Rows>(lane, wave);
  f32x16 dka[kKB][G::kDB], dva[kKB][G::kDB];               // set by the first step

  const int n_steps = (n_qrows + kW64Rows - 1) / kW64Rows;
  // Loads of tile t: the row statistics first and scaled only when
  // committed, so no wait for them covers the tile loads.
  float st_lse = 0.0f, st_d = 0.0f;
  auto issue = [&](int t, uint32_t stage) {
    const int q0 = t * kW64Rows;
    if (tid < kW64Rows) {
      const int row = q0 + tid;
      st_lse = row < n_qrows ? lse[head_q + row] : INFINITY;
      st_d = row < n_qrows ? dvec[head_q + row] : 0.0f;
    }
    dma_tile<D, kW64Rows>(q + head_q * D, q0, n_qrows, stage, wave, off.dvoff);
    dma_tile<D, kW64Rows>(dout + head_q * D, q0, n_qrows, stage + kTileB, wave, off.dvoff);
  };
  auto commit = [&](uint32_t stage) {
    if (tid < kW64Rows) {
      *(__attribute__((address_space(3))) float*)(uintptr_t)(stage + 2 * kTileB + tid * 4) = st_lse * kLog2e;
      *(__attribute__((address_space(3))) float*)(uintptr_t)(stage + 2 * kTileB + kW64Rows * 4 + tid * 4) = st_d;
    }
  };
  // Per-lane LDS offsets.  The tile swizzle is an XOR on the 16-byte chunk
  // index, so k-step s of a row read sits at row0 ^ 32 s and d block db of
  // a transposing read at tr0 ^ 64 db (rows +0..3) and its ^ kTrX, + 16 D
  // (rows +8..11: one more swizzle bit): two registers instead of up to
  // sixteen, one XOR per read.
  constexpr int kTrX = D == 128 ? 128 : 16;
  int row0 = off.row[0], tr0 = off.tr[0];
  auto R = [&](uint32_t tile, int s) { return lds_row(tile, row0 ^ (32 * s)); };
  auto T = [&](uint32_t tile, int s2, int db) {
    const int lo = tr0 ^ (64 * db);
    return lds_tr(tile + (uint32_t)(16 * s2 * D * 2), lo, (lo ^ kTrX) + 16 * D);
  };
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

  issue(0, lds);
  // K, V and tile 0 have landed
  wait_vm();
  commit(lds);
  __syncthreads();

  // One query tile per step, stage t % 2 (a compile-time constant: the loop
  // runs two steps per trip).  The step's instructions are placed in a
  // fixed order (fences between groups) so that each product's operand is
  // read two products ahead and the vector work runs between the products
  // that do not depend on it:
  //   1. S = Q K^T                      (16 products)
  //   2. dP = dO V^T, and P = exp2(S c - lse) in place   (16 products)
  //   3. dV^T += dO^T P, and dS = P (dP - D) packed      (16 products)
  //   4. dK^T += Q^T dS                                  (16 products)
  auto step = [&](const int t, auto stage_c, auto first_c) {
    constexpr int st = decltype(stage_c)::value;
    constexpr bool first = decltype(first_c)::value;
    const uint32_t stage = lds + (uint32_t)st * kStageB;
    const uint32_t qtile = stage, dotile = stage + kTileB;
    const uint32_t lse_s = stage + 2 * kTileB, d_s = lse_s + kW64Rows * 4;
    const bool more = t + 1 < n_steps;
    if (more) issue(t + 1, lds + (uint32_t)(1 - st) * kStageB);
    // recomputed each step, not kept as sixteen loop-invariant registers
    asm volatile("" : "+v"(row0), "+v"(tr0));
    fence();
    f32x16 sacc[kKB], pacc[kKB];
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) sacc[kb] = pacc[kb] = f32x16{};
    // 1. S
    bf16x8 a[G::kKSteps];
    a[0] = R(qtile, 0);
    a[1] = R(qtile, 1);
    fence();
    f32x4 l4[4];
#pragma unroll
    for (int s = 0; s < G::kKSteps; ++s) {
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) sacc[kb] = mfma32x32x16(a[s], kf[kb][s], sacc[kb]);
      if (s + 2 < G::kKSteps) a[s + 2] = R(qtile, s + 2);
      else a[s + 2 - G::kKSteps] = R(dotile, s + 2 - G::kKSteps);
      if (s == G::kKSteps - 4) l4[0] = *(const lds_f32x4*)(uintptr_t)(lse_s + 4 * hh * 4);
      if (s == G::kKSteps - 3) l4[1] = *(const lds_f32x4*)(uintptr_t)(lse_s + (8 + 4 * hh) * 4);
      fence();
    }
    // 2. dP, with the weights P = exp2(S c - lse) in place (lse of rows r
    // read two units ahead) and the bf16 packing of rows 0 and 1 in the
    // second half: after each product a slot of vector work, so it issues
    // while the product runs (a second product right behind the first would
    // hold the wave until the first is done).  Slot i takes the kEPS values
    // e = i kEPS .. of the 32 a lane holds: block kb = (e / 4) % 2, rows
    // r = e / 8 (8 r + 4 hh + e % 4 of the tile).
    f32x4 d4[4];
    u32x4 pu[2][kKB];
#pragma unroll
    for (int s = 0; s < G::kKSteps; ++s) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = 2 * s + h;
        pacc[h] = mfma32x32x16(a[s], vf[h][s], pacc[h]);
        fence();
#pragma unroll
        for (int k = 0; k < kEPS; ++k) {
          const int e = i * kEPS + k, r = e / 8, kb = (e / 4) % 2, j = e % 4;
          sacc[kb][4 * r + j] = exp2_fast(__builtin_fmaf(sacc[kb][4 * r + j], c_log2, -l4[r][j]));
        }
        if (i >= kNS / 2) {
#pragma unroll
          for (int k = 0; k < 16 / kNS; ++k) {
            const int wi = (i - kNS / 2) * (16 / kNS) + k, kb = wi / 4, w = wi % 4;
            pu[0][kb][w] = pack_bf16x2(sacc[kb][2 * w], sacc[kb][2 * w + 1]);
          }
        }
        {
          const int e0 = i * kEPS, r = e0 / 8;
          if (e0 % 8 == 0 && r + 2 < 4) l4[r + 2] = *(const lds_f32x4*)(uintptr_t)(lse_s + (8 * (r + 2) + 4 * hh) * 4);
        }
        if (h == 1) {
          if (s + 2 < G::kKSteps) a[s + 2] = R(dotile, s + 2);
          if (s == G::kKSteps - 2) d4[0] = *(const lds_f32x4*)(uintptr_t)(d_s + 4 * hh * 4);
          if (s == G::kKSteps - 1) d4[1] = *(const lds_f32x4*)(uintptr_t)(d_s + (8 + 4 * hh) * 4);
        }
        fence();
      }
    }
    // 3. dV, with dS = P (dP - D) formed and packed in slots as above
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        pu[1][kb][w] = pack_bf16x2(sacc[kb][8 + 2 * w], sacc[kb][8 + 2 * w + 1]);
    bf16x8 tb[2];
    tb[0] = T(dotile, 0, 0);
    tb[1] = T(dotile, 0, 1);
    fence();
    u32x4 du[2][kKB];
#pragma unroll
    for (int g = 0; g < 2 * G::kDB; ++g) {
      const int s2 = g / G::kDB, db = g % G::kDB;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = 2 * g + h;
        // only the first product follows the packing of P closely
        if (first && s2 == 0) {
          if (g == 0 && h == 0) mfma_agpr_first<true>(dva[h][db], tb[g % 2], as_bf16x8(pu[s2][h]));
          else mfma_agpr_first<false>(dva[h][db], tb[g % 2], as_bf16x8(pu[s2][h]));
        } else {
          if (g == 0 && h == 0) mfma_agpr<true>(dva[h][db], tb[g % 2], as_bf16x8(pu[s2][h]));
          else mfma_agpr<false>(dva[h][db], tb[g % 2], as_bf16x8(pu[s2][h]));
        }
        fence();
        {
          const int e0 = i * kEPS, r = e0 / 8;
          if (e0 % 8 == 0 && r + 2 < 4) d4[r + 2] = *(const lds_f32x4*)(uintptr_t)(d_s + (8 * (r + 2) + 4 * hh) * 4);
        }
#pragma unroll
        for (int k = 0; k < kEPS; k += 2) {
          const int e = i * kEPS + k, r = e / 8, kb = (e / 4) % 2, j = e % 4;
          const float ds0 = sacc[kb][4 * r + j] * (pacc[kb][4 * r + j] - d4[r][j]);
          const float ds1 = sacc[kb][4 * r + j + 1] * (pacc[kb][4 * r + j + 1] - d4[r][j + 1]);
          // rows r = 2 s2' + q: packed word 2 q + j / 2 of du[s2'][kb]
          du[r / 2][kb][2 * (r % 2) + j / 2] = pack_bf16x2(ds0, ds1);
        }
        if (h == 1) {
          if (g + 2 < 2 * G::kDB) tb[g % 2] = T(dotile, (g + 2) / G::kDB, (g + 2) % G::kDB);
          else tb[g % 2] = T(qtile, (g + 2 - 2 * G::kDB) / G::kDB, (g + 2 - 2 * G::kDB) % G::kDB);
        }
        fence();
      }
    }
    // 4. dK (each dS word was packed at least four products before its
    // first use)
#pragma unroll
    for (int g = 0; g < 2 * G::kDB; ++g) {
      const int s2 = g / G::kDB, db = g % G::kDB;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        if (first && s2 == 0) mfma_agpr_first<false>(dka[kb][db], tb[g % 2], as_bf16x8(du[s2][kb]));
        else mfma_agpr<false>(dka[kb][db], tb[g % 2], as_bf16x8(du[s2][kb]));
      }
      if (g + 2 < 2 * G::kDB) tb[g % 2] = T(qtile, (g + 2) / G::kDB, (g + 2) % G::kDB);
      fence();
    }
    // unconditional: the compiler then knows no load is in flight at the
    // next step's start (else it waits for the next tile's loads there)
    wait_vm();
    if (more) commit(lds + (uint32_t)(1 - st) * kStageB);
    __syncthreads();
  };
  step(0, std::integral_constant<int, 0>{}, std::true_type{});
  for (int t = 1; t < n_steps; t += 2) {
    step(t, std::integral_constant<int, 1>{}, std::false_type{});
    if (t + 1 < n_steps) step(t + 1, std::integral_constant<int, 0>{}, std::false_type{});
  }

  // The compiler does not see the products above as matrix-core work:
  // wait out their write latency (18 wait states) before the accumulators
  // are read, each accumulator passing through an (empty) statement ordered
  // after the wait.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
    for (int i = 0; i < G::kDB; ++i) {
      asm volatile("" : "+a"(dka[kb][i]));
      asm volatile("" : "+a"(dva[kb][i]));
    }
  // dV, then dK, through LDS: the accumulators hold four consecutive d of a
  // row per lane, so direct stores would complete each 256-byte row with 16
  // partial writes, and with 128 KB of output per workgroup the L2 evicts
  // lines before they are whole (measured: 2.3x the bytes).  Each wave
  // writes its 64 rows to its own 16 KB of LDS (16-byte chunks XOR-swizzled
  // by row), then stores whole rows, D / 8 lanes per row.  The last step's
  // barrier has freed the tile stages; one wave's LDS accesses stay in
  // order, so dK may overwrite dV's rows once they are read.
  const uint32_t wout = lds + (uint32_t)wave * kOutB;
  auto store_out = [&](f32x16 (&acc)[kKB][G::kDB], float mul, __bf16* __restrict__ out) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int db = 0; db < G::kDB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // key 32 kb + l32, d = 32 db + 8 r + 4 hh .. + 3: 16-byte chunk 4 db + r
          const int row = 32 * kb + l32;
          u32x2 w;
          w[0] = pack_bf16x2(acc[kb][db][4 * r + 0] * mul, acc[kb][db][4 * r + 1] * mul);
          w[1] = pack_bf16x2(acc[kb][db][4 * r + 2] * mul, acc[kb][db][4 * r + 3] * mul);
          *(__attribute__((address_space(3))) u32x2*)(uintptr_t)(
              wout + (uint32_t)(row * D * 2 + (((4 * db + r) ^ (row & (G::kCPR - 1))) * 16) + hh * 8)) = w;
        }
    const int c = lane % G::kCPR;
#pragma unroll
    for (int i = 0; i < kW64Keys * G::kCPR / kWave; ++i) {
      const int row = (kWave / G::kCPR) * i + lane / G::kCPR;
      const u32x4 v16 = *(const lds_u32x4*)(uintptr_t)(wout + (uint32_t)(row * D * 2 + ((c ^ (row & (G::kCPR - 1))) * 16)));
      const int key = kt * kW64WgKeys + wave * kW64Keys + row;
      if (key < N) *reinterpret_cast<u32x4*>(out + (head_kv + key) * D + c * 8) = v16;
    }
  };
  store_out(dva, 1.0f, dv);
  store_out(dka, scale, dk);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup of kW waves per kW * 32 query rows of head (b, h), R-key
// tiles.  Each K / V tile is loaded once per workgroup (by its first kBWaves
// waves) and read by all kW: at kW = 8, two waves per SIMD as with two 4-wave
// workgroups, half the tile loads per query row (measured 1.2 - 1.5 % faster
// backward at d = 128, bit-identical).
constexpr int kDqWaves = 8;
// keys per LDS tile: 128 at d = 64 (halves the barriers; measured 0.6 %
// faster), 64 at d = 128 (the 128 KB of two 128-key stages measured slower)
template <int D>
constexpr int kDqTRows = D == 128 ? kTRows : 2 * kTRows;

template <int D, int kW, int R>
__global__ __launch_bounds__(kW * kWave, 8 / kW)
void attn_bwd_dq_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                        const __bf16* __restrict__ v, const __bf16* __restrict__ o,
                        const __bf16* __restrict__ dout, const float* __restrict__ lse,
                        float* __restrict__ dvec,
                        __bf16* __restrict__ dq, int Hq, int Hkv, int N, float c_log2, float scale,
                        int n_qtiles, uint32_t n_xcd) {
  using G = BGeo<D, R>;
  constexpr uint32_t kTileB = G::kTile * 2;
  constexpr uint32_t kStageB = 2 * kTileB;          // K tile, V tile
  __shared__ __align__(16) unsigned char smem[2 * kStageB];
  const uint32_t lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // query tiles over the group's (Hq / Hkv) * N adjacent rows, numbered
  // fastest (as the forward)
  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x, n_xcd);
  const int qt = (int)(logical % (uint32_t)n_qtiles);
  const uint32_t rest = logical / (uint32_t)n_qtiles;
  const int kvh = (int)(rest % (uint32_t)Hkv);
  const int b = (int)(rest / (uint32_t)Hkv);
  const int n_qrows = (Hq / Hkv) * N;
  const int64_t head_q = ((int64_t)b * Hkv + kvh) * (int64_t)n_qrows;
  const int64_t head_kv = ((int64_t)b * Hkv + kvh) * (int64_t)N;
  const __bf16* kh = k + head_kv * D;
  const __bf16* vh = v + head_kv * D;

  static_assert(kW % kBWaves == 0, "tile loads split over the first kBWaves waves");
  const bool loader = wave < kBWaves;   // wave-uniform
  const TileOffsets<D, R> off = tile_offsets<D, R>(lane, wave % kBWaves);
  if (loader) {
    dma_tile<D, R>(kh, 0, N, lds, wave, off.dvoff);
    dma_tile<D, R>(vh, 0, N, lds + kTileB, wave, off.dvoff);
  }

  const int qrow = qt * kW * kWRows + wave * kWRows + l32;   // this lane's query
  const bool qvalid = qrow < n_qrows;
  bf16x8 qf[G::kKSteps], df[G::kKSteps];
  load_rowfrags<D>(qf, q + head_q * D, qrow, n_qrows, hh);
  load_rowfrags<D>(df, dout + head_q * D, qrow, n_qrows, hh);
  const int qr = min(qrow, n_qrows - 1);
  const float lse2 = lse[head_q + qr] * kLog2e;
  // D of this lane's query row, dO . O in fp32: this lane's half of d
  // (the dO fragments it holds), then the other half-wave's (lane ^ 32);
  // written for the dK/dV kernel, which runs after this one
  float dpart = 0.0f;
  {
    const __bf16* po = o + (head_q + qr) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < G::kKSteps; ++s) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(po + 16 * s);
      const u32x4 b = __builtin_bit_cast(u32x4, df[s]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dpart = __builtin_fmaf(bf16_bits_to_float(a[w] & 0xFFFFu), bf16_bits_to_float(b[w] & 0xFFFFu), dpart);
        dpart = __builtin_fmaf(bf16_bits_to_float(a[w] >> 16), bf16_bits_to_float(b[w] >> 16), dpart);
      }
    }
  }
  const float dd = dpart + __shfl_xor(dpart, 32);
  if (qvalid && hh == 0) dvec[head_q + qrow] = dd;

  f32x16 dqacc[G::kDB];
#pragma unroll
  for (int i = 0; i < G::kDB; ++i) dqacc[i] = f32x16{};

  wait_vm();
  __syncthreads();

  const int n_kt = (N + R - 1) / R;
  // one key tile in LDS stage `st` (a compile-time constant: the loop below
  // runs two tiles per trip, so every LDS read has a fixed offset)
  auto key_tile = [&](const int jt, auto stage_c) {
    constexpr int st = decltype(stage_c)::value;
    const uint32_t ktile = lds + (uint32_t)st * kStageB, vtile = ktile + kTileB;
    if (loader && jt + 1 < n_kt) {
      const uint32_t nxt = lds + (uint32_t)(1 - st) * kStageB;
      dma_tile<D, R>(kh, (jt + 1) * R, N, nxt, wave, off.dvoff);
      dma_tile<D, R>(vh, (jt + 1) * R, N, nxt + kTileB, wave, off.dvoff);
    }
#pragma unroll
    for (int kb = 0; kb < R / 32; ++kb) {
      // S^T = K Q^T and dP^T = V dO^T: 32 keys x this wave's 32 queries
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int s = 0; s < G::kKSteps; ++s) {
        const bf16x8 ka = lds_row(ktile + kb * 32 * D * 2, off.row[s]);
        const bf16x8 va = lds_row(vtile + kb * 32 * D * 2, off.row[s]);
        sacc = mfma32x32x16(ka, qf[s], sacc);
        pacc = mfma32x32x16(va, df[s], pacc);
      }
      // Keys past N need no mask: their K and V rows read as zeros, so their
      // dS meets a zero row of K in dQ += K^T dS^T.  Their weight 2^-lse2
      // only has to stay finite, which the clamp of every weight to [0, 1]
      // (the exponent's output modifier; a weight of a key that exists is
      // at most 1 up to rounding) guarantees.
      float ds[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = __builtin_amdgcn_fmed3f(exp2_fast(__builtin_fmaf(sacc[e], c_log2, -lse2)), 0.0f, 1.0f);
        ds[e] = pe * (pacc[e] - dd);
      }
      // dQ^T += K^T dS^T over the two 16-key k-steps
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 du;
#pragma unroll
        for (int w = 0; w < 4; ++w) du[w] = pack_bf16x2(ds[8 * s2 + 2 * w], ds[8 * s2 + 2 * w + 1]);
        const uint32_t rb = (uint32_t)((kb * 32 + 16 * s2) * D * 2);
#pragma unroll
        for (int db = 0; db < G::kDB; ++db)
          dqacc[db] = mfma32x32x16(lds_tr(ktile + rb, off.tr[db], off.tr8[db]), as_bf16x8(du), dqacc[db]);
      }
    }
    wait_vm();
    __syncthreads();
  };
  for (int jt = 0; jt < n_kt; jt += 2) {
    key_tile(jt, std::integral_constant<int, 0>{});
    if (jt + 1 < n_kt) key_tile(jt + 1, std::integral_constant<int, 1>{});
  }

  if (qvalid) store_rowT<D>(dqacc, dq + (head_q + qrow) * D, scale, hh);
}

template <int D>
hipError_t launch_d(const FwdArgs& a, const BwdArgs& g) {
  const float c_log2 = a.scale * kLog2e;
  // dQ first: it also writes D (the dK/dV kernel's input)
  constexpr int kDqRows = kDqWaves * kWRows;
  const int n_qt = (int)(((uint64_t)(a.Hq / a.Hkv) * a.N + kDqRows - 1) / kDqRows);
  const uint64_t grid2 = (uint64_t)n_qt * a.Hkv * a.B;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, kDqWaves, kDqTRows<D>>), dim3((uint32_t)grid2),
                     dim3(kDqWaves * kWave), 0, a.stream, static_cast<const __bf16*>(a.q),
                     static_cast<const __bf16*>(a.k), static_cast<const __bf16*>(a.v),
                     static_cast<const __bf16*>(a.o), static_cast<const __bf16*>(g.dout), a.lse,
                     g.dvec, static_cast<__bf16*>(g.dq), a.Hq, a.Hkv, a.N, c_log2, a.scale, n_qt,
                     (uint32_t)a.n_xcd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // head dim 128: one wave per 64 keys (attn_bwd_dkdv_w64_kernel); 64: two
  // waves per SIMD of 32 keys each (attn_bwd_dkdv_kernel: the one-wave form
  // ran 4 % slower there, its step bound by vector work that a second wave
  // no longer hides)
  const int wg_keys = D == 128 ? kW64WgKeys : kWgRows;
  const int n_kt = (a.N + wg_keys - 1) / wg_keys;
  const uint64_t grid1 = (uint64_t)n_kt * a.Hkv * a.B;
  if constexpr (D == 128) {
    hipLaunchKernelGGL((attn_bwd_dkdv_w64_kernel<D>), dim3((uint32_t)grid1), dim3(kBThreads), 0,
                       a.stream, static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                       static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(g.dout), a.lse,
                       g.dvec, static_cast<__bf16*>(g.dk), static_cast<__bf16*>(g.dv), a.Hq, a.Hkv,
                       a.N, c_log2, a.scale, n_kt, (uint32_t)a.n_xcd);
  } else {
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D>), dim3((uint32_t)grid1), dim3(kBThreads), 0,
                       a.stream, static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                       static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(g.dout), a.lse,
                       g.dvec, static_cast<__bf16*>(g.dk), static_cast<__bf16*>(g.dv), a.Hq, a.Hkv,
                       a.N, c_log2, a.scale, n_kt, (uint32_t)a.n_xcd);
  }
  return hipGetLastError();
}

}  // namespace

// An upper bound of every backward grid (128 rows per workgroup).
uint64_t bwd_grid(int B, int Hq, int Hkv, int N) {
  return ((uint64_t)(Hq / Hkv) * N + kWgRows - 1) / kWgRows * Hkv * B;
}

hipError_t launch_bwd_bf16(const FwdArgs& a, const BwdArgs& g) {
  return a.d == 128 ? launch_d<128>(a, g) : launch_d<64>(a, g);
}

}  // namespace attn
