// rows64_pipeline.hpp -- the d = 128 (and 64) fused forward kernel body,
// shared by two translation units: attn_fwd_bf16_rows64.hip (ATTN_ROWS64_SPLIT
// 0: every key of a head; the attn_fwd path) and attn_fwd_bf16_split.hip (1:
// one key range per workgroup, partial results to a workspace; the
// attn_fwd_split path).  The switch only adds code, so the attn_fwd kernel
// is compiled from exactly the text it would be on its own.
//
// bf16 I/O, two 32-row query blocks per wave (used for head dim 128).
//
// The IO-aware forward (blog "attention 的显存线性化", section 三; the
// "efficient attention" chapter's online-softmax paragraph): one workgroup
// owns kFBr query rows of one head and streams every key/value tile of that
// head through LDS, keeping per row a running maximum m and exp-sum l and
// an fp32 output accumulator.  S and P only ever exist in registers.
//
// Design for CDNA4:
//  * 4 waves x 64 query rows (two 32-row blocks per wave).  Each wave
//    computes S^T = K Q^T per 32-key tile with v_mfma_f32_32x32x16_bf16 (K
//    from LDS as the A operand, the wave's Q rows resident in VGPRs as the B
//    operand).  Every K fragment read from LDS feeds both query blocks, and
//    likewise every V fragment below, which halves the LDS traffic per FLOP
//    against one block per wave (LDS read bandwidth, not the matrix cores,
//    limits that layout).
//  * In the S^T output layout a lane owns ONE query (column l % 32) and 16
//    of the 32 keys, so the row max / row sum are in-lane reductions plus
//    one v_permlane32_swap with the other half-wave.  The swap is needed
//    only when the running max moves: whether it must is a ballot of each
//    half-row's own max.
//  * O^T = V^T P^T on the same MFMA: P^T comes straight from the S^T
//    accumulator registers (rounded to bf16); the V^T operand is read from
//    the row-major V tile with ds_read_b64_tr_b16, which hands each lane
//    four consecutive keys of one d column.  The O^T accumulator again gives
//    each lane one query, so the rescale by exp(m_old - m_new) is a per-lane
//    scalar.
//  * Software pipeline across key tiles: step j issues the Q K^T products
//    of tile j+1 and the P V products of tile j-1 while it runs the softmax
//    of tile j.  The step is scheduled by hand: every MFMA is followed by a
//    slice of the softmax work, the slices balanced by their cycle cost, and
//    a scheduling fence keeps that order, so one wave keeps the matrix core
//    and the vector ALU busy at the same time.  With one wave per SIMD every
//    instruction it issues between two MFMAs costs time (~4 cycles each,
//    measured), so the step carries as few as it can: the rare rescale in a
//    wave-uniform branch, tile-load addresses advanced rather than rebuilt.
//  * K and V tiles go global -> LDS directly (buffer_load ... lds, the rows
//    past N read as zeros by the buffer's range check) into a ring of four
//    slots each, three tiles ahead of their use; one barrier per step.  The
//    slot of every access is a compile-time constant (the step loop is
//    unrolled by the ring size).  Rows sit unpadded with their 16-byte
//    chunks XOR-swizzled by the row index, so both the MFMA operand reads of
//    K and the transposing reads of V are free of LDS bank conflicts.
//  * The scale is folded into exp2: p = 2^(s * scale * log2 e - m).  The
//    running max is only moved when some row's max grows by more than
//    kRescaleLog2 (softmax is unchanged by any common shift of a row, the
//    basis of the rescale rule), so the rescale of the accumulator is rare.
//  * Workgroups of one K/V head are numbered consecutively and remapped so
//    they run on one XCD and share its L2.  One XCD holds 32 x 256 query rows
//    at a time, so a head with more query rows streams its K/V through that
//    L2 once per round of workgroups.  Where a head's K/V fits the L2, every
//    other round streams the keys in reverse order, so it starts on the tiles
//    the round before left in the L2 (the result is the same up to the
//    rounding order), and O is stored as whole rows through LDS with a
//    non-temporal hint; Q is always loaded with one.  Neither then displaces
//    K/V from the L2, and no O line is written back in pieces.
#pragma once

#ifndef ATTN_ROWS64_SPLIT
#error "define ATTN_ROWS64_SPLIT (0 or 1) before including rows64_pipeline.hpp"
#endif
#if ATTN_ROWS64_SPLIT
#define ATTN_KEYS Nk     // keys of this workgroup's range
#else
#define ATTN_KEYS N      // every key of the head
#endif

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <utility>

#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kFWaves = 4;
constexpr int kFThreads = kFWaves * kWave;
constexpr int kQB = 2;                       // 32-row query blocks per wave
constexpr int kFRows = 32 * kQB;             // query rows per wave
constexpr int kFBr = kFWaves * kFRows;       // query rows per workgroup
constexpr int kBc = 32;                      // keys per tile
constexpr int kSlots = 4;                    // LDS ring depth per K and V
constexpr float kRescaleLog2 = 8.0f;         // move m only when it grows by > 2^8

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) void lds_void;

template <int D>
struct FGeo {
  static constexpr int kKSteps = D / 16;               // MFMA k-steps over d
  static constexpr int kDB = D / 32;                   // 32-wide d blocks
  static constexpr int kCPR = D / 8;                   // 16-byte chunks per row
  static constexpr int kTile = kBc * D;                // bf16 elements of one K (or V) tile
  static constexpr int kDma = kTile / 8 / kFThreads;   // 16-B loads per lane per tile
  static constexpr int kUnits = kKSteps;               // (K frag, V frag) pairs per step
  static_assert(kDma * 8 * kFThreads == kTile, "tile must split over the workgroup");
  static_assert(kCPR >= 8, "the chunk swizzle needs at least 8 chunks per row");
  static_assert(2 * kDB == kUnits, "one V^T fragment per K fragment");
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

// IEEE-754 maximum / minimum (v_maximum3_f32 / v_minimum3_f32 on gfx950):
// unlike fmaxf they need no canonicalisation of MFMA results first.
template <bool kNeg>
__device__ __forceinline__ float ext2(float a, float b) {
  return kNeg ? __builtin_elementwise_minimum(a, b) : __builtin_elementwise_maximum(a, b);
}
template <bool kNeg>
__device__ __forceinline__ float ext3(float a, float b, float c) {
  return ext2<kNeg>(ext2<kNeg>(a, b), c);
}

// Across the two half-waves (lane l and l ^ 32): both get the combined value.
template <bool kNeg>
__device__ __forceinline__ float xhalf_ext(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return ext2<kNeg>(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// acc += a b with the accumulator in AGPRs, so the P V products leave the
// VGPR ports to the softmax beside them (3.5 - 4 % faster than the
// compiler's VGPR-form product).  The compiler does not see these as
// matrix-core work, so every vector-ALU access to an accumulator it makes
// must follow the product's write latency: kPad products wait it out
// themselves (the last tile's, where the compiler moves accumulators
// between registers), and oacc_settle waits before the other reads.  A
// matrix-core read of a register the vector ALU wrote needs two wait
// states (the s_nop 1; every b here was written at least that early
// otherwise); back-to-back products into one accumulator need none.
template <bool kPad>
__device__ __forceinline__ void mfma_oacc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (kPad)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <int NQ, int ND>
__device__ __forceinline__ void oacc_settle(f32x16 (&o)[NQ][ND]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < NQ; ++i)
#pragma unroll
    for (int j = 0; j < ND; ++j) asm volatile("" : "+a"(o[i][j]));
}

// ---------------------------------------------------------------------------
// Per-wave state.
template <int D>
struct WaveState {
  using G = FGeo<D>;
  bf16x8 qf[kQB][G::kKSteps];      // Q^T operands, resident
  f32x16 oacc[kQB][G::kDB];        // O^T accumulators
  f32x16 s[2][kQB];                // S^T of a tile, by tile parity
  u32x4 p[2][kQB][2];              // bf16 P^T operands [parity][query block][16-key half]
  float m[kQB];                    // running max of the log2-scaled scores (per lane's query)
  float l[kQB];                    // this lane's part of the exp-sum
  int koff[G::kKSteps];            // LDS byte offsets of the K operand reads
  int voff[G::kDB];                // LDS byte offsets of the V^T transposing reads (rows +0..3)
  int voff8[D == 128 ? 1 : G::kDB];  // the same for rows +8..11 (d = 64 only, see hi_off)
  int dvoff[G::kDma];              // byte offsets of this lane's direct loads within a tile
  int rev_last;                    // > 0: keys run in reverse order; the first key of the last tile
  const char* kp;                  // byte address of the next K tile to load
  const char* vp;                  // the same for V
  int kleft, vleft;                // keys from the first key of that tile to the end
  int dleft;                       // change of kleft / vleft per tile (-kBc, or kBc in reverse)
};

// Byte offset of the transposing V read of rows +8..11 for d block db.  For
// d = 128, swz(r + 8) = swz(r) ^ 8 for r < 8 and bit 3 of the lane's chunk is
// db / 2, so the offset differs from rows +0..3 by a constant.
template <int D>
__device__ __forceinline__ int hi_off(const WaveState<D>& w, int db) {
  if (D == 128) return w.voff[db] + 8 * D * 2 + ((db >> 1) ? -128 : 128);
  return w.voff8[db];
}

// The tile loads: the next tile of one stream (K or V) in this wave's key
// order into one LDS slot.  Each stream keeps the byte address of its next
// tile and the keys from that tile's first key to the end of the range
// ("left"), moved by one tile per load (backwards in reverse order).  The
// buffer covers only the tile's rows that exist, so rows past the end read
// as zeros and a tile outside the range (left <= 0, or left > N once a
// reverse-order wave has passed the first key) reads nothing; every operand
// of the buffer resource is wave-uniform (SGPRs).  Issued as inline
// assembly: the compiler then does not see an LDS write in flight and does
// not stall the LDS reads of the other slots behind it; the step's own
// vmcnt wait and barrier order these loads against readers.
template <int D>
__device__ __forceinline__ void dma_next(const int* dvoff, const char*& ptr, int& left, int dleft,
                                         int N, uint32_t lds_byte, int wave) {
  using G = FGeo<D>;
  // 0 < left <= N, as one unsigned compare
  const int rows = (uint32_t)(left - 1) < (uint32_t)N ? (left < kBc ? left : kBc) : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(ptr), (short)0, rows * D * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < G::kDma; ++i) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(
        lds_byte + (uint32_t)((wave * G::kDma + i) * kWave * 16));
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 ::"s"(dst), "v"(dvoff[i]), "s"(rs) : "memory");
  }
  ptr -= (int64_t)dleft * (D * 2);
  left += dleft;
}

__device__ __forceinline__ bf16x8 lds_k(uint32_t base, int off) {
  const u32x4 u = *(const lds_u32x4*)(uintptr_t)(base + off);
  return as_bf16x8(u);
}

__device__ __forceinline__ bf16x8 lds_vt(uint32_t base, int off, int off8) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(base + off));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(base + off8));
  const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, a8);
}

// ---------------------------------------------------------------------------
// The softmax of one tile as a list of small tasks, run in order and spread
// over the MFMA slots of a step by their cost.
//   tasks 0 .. 17   : row max, 9 per query block; the ninth tests the lane's
//                     half-row max against m + kRescaleLog2 (a ballot)
//   task  18        : if any lane's test fired (a wave-uniform branch): the
//                     max over both half-rows, the new m, alpha, l *= alpha
//   tasks 19 .. 34  : 2 weights each: fma, exp2, add to l, round to bf16
//   task  35        : fold the partial sums into l
constexpr int kMaxTasks = 9;
constexpr int kTasks = 2 * kMaxTasks + 1 + 16 + 1;

// Approximate VALU cycles of each task (full-rate op 2, transcendental 8).
__host__ __device__ constexpr int task_cost(int t) {
  return t < 2 * kMaxTasks ? ((t % kMaxTasks) == kMaxTasks - 1 ? 8 : 2)
       : t == 2 * kMaxTasks ? 36
       : t < kTasks - 1 ? 26
       : 8;
}
__host__ __device__ constexpr int task_cost_sum(int n) {
  int c = 0;
  for (int t = 0; t < n; ++t) c += task_cost(t);
  return c;
}
// First task of slot i when kTasks tasks are spread over n_slots slots.
__host__ __device__ constexpr int task_begin(int i, int n_slots) {
  if (i >= n_slots) return kTasks;
  const int target = (task_cost_sum(kTasks) * i + n_slots - 1) / n_slots;
  int t = 0;
  while (t < kTasks && task_cost_sum(t) < target) ++t;
  return t;
}

// Task ranges of every slot, as a table of compile-time constants.
template <int NS>
struct TaskSplit {
  int b[NS + 1];
  constexpr TaskSplit() : b() {
    for (int i = 0; i <= NS; ++i) b[i] = task_begin(i, NS);
  }
};

struct SoftmaxScratch {
  float mx[kQB][7];
  float ext[kQB];
  float alpha[kQB];
  uint64_t hit[kQB];
  float ls[kQB][2];
  bool need;
};

template <int D, bool kNeg, bool kMask, int kPar>
__device__ __forceinline__ void softmax_task(int t, WaveState<D>& w, SoftmaxScratch& sc,
                                             float c_log2, int valid, int hh) {
  const float kFill = kNeg ? INFINITY : -INFINITY;
  if (t < 2 * kMaxTasks) {
    const int qb = t / kMaxTasks;
    const int i = t % kMaxTasks;
    const f32x16& a = w.s[kPar][qb];
    // element e of a lane holds key 8 (e / 4) + 4 hh + e % 4 of the tile
    auto val = [&](int e) {
      if (!kMask) return a[e];
      return (8 * (e >> 2) + 4 * hh + (e & 3)) < valid ? a[e] : kFill;
    };
    if (i < 5) {
      sc.mx[qb][i] = ext3<kNeg>(val(3 * i), val(3 * i + 1), val(3 * i + 2));
    } else if (i == 5) {
      sc.mx[qb][5] = ext3<kNeg>(sc.mx[qb][0], sc.mx[qb][1], val(15));
    } else if (i == 6) {
      sc.mx[qb][6] = ext3<kNeg>(sc.mx[qb][2], sc.mx[qb][3], sc.mx[qb][4]);
    } else if (i == 7) {
      sc.mx[qb][5] = ext2<kNeg>(sc.mx[qb][5], sc.mx[qb][6]);
    } else {
      sc.hit[qb] = __builtin_amdgcn_ballot_w64(
          __builtin_fmaf(sc.mx[qb][5], c_log2, -w.m[qb]) > kRescaleLog2);
    }
  } else if (t == 2 * kMaxTasks) {
    // move the running max only when some row's max grows by > 2^kRescaleLog2
    sc.need = (sc.hit[0] | sc.hit[1]) != 0;
    if (sc.need) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        sc.ext[qb] = xhalf_ext<kNeg>(sc.mx[qb][5]) * c_log2;   // the row's max of s * c_log2
        const float m_new = __builtin_fmaxf(w.m[qb], sc.ext[qb]);
        sc.alpha[qb] = exp2_fast(w.m[qb] - m_new);   // 0 on the first tile
        w.m[qb] = m_new;
        w.l[qb] *= sc.alpha[qb];
      }
    }
  } else if (t < kTasks - 1) {
    const int kk = t - (2 * kMaxTasks + 1);   // 0 .. 15
    const int qb = kk / 8;
    const int x = kk % 8;                     // weight pair: elements 2x, 2x + 1
    const f32x16& a = w.s[kPar][qb];
    float p0 = exp2_fast(__builtin_fmaf(a[2 * x], c_log2, -w.m[qb]));
    float p1 = exp2_fast(__builtin_fmaf(a[2 * x + 1], c_log2, -w.m[qb]));
    if (kMask) {
      const int e0 = 2 * x, e1 = 2 * x + 1;
      if (8 * (e0 >> 2) + 4 * hh + (e0 & 3) >= valid) p0 = 0.0f;
      if (8 * (e1 >> 2) + 4 * hh + (e1 & 3) >= valid) p1 = 0.0f;
    }
    // l sums the fp32 weights: the bf16-rounded ones would cost lse about
    // half a bf16 ulp of relative error on short rows
    if (x == 0) {
      sc.ls[qb][0] = p0;
      sc.ls[qb][1] = p1;
    } else {
      sc.ls[qb][0] += p0;
      sc.ls[qb][1] += p1;
    }
    // P^T slot (hh, e) of k-step s2 holds key 16 s2 + 8 (e / 4) + 4 hh + e % 4,
    // i.e. elements 8 s2 .. 8 s2 + 7 of the S^T accumulator
    w.p[kPar][qb][x / 4][x % 4] = pack_bf16x2(p0, p1);
  } else {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) w.l[qb] += sc.ls[qb][0] + sc.ls[qb][1];
  }
}

// ---------------------------------------------------------------------------
// One pipeline step j (kJ4 = j mod kSlots; the slot of every LDS access is
// a compile-time constant, which the scheduler and register allocator need):
//   * loads K tile j + S and V tile j + S - 2 into the slots freed last step
//     (S = kSlots; K tile t lives in K slot t % S, V tile t in V slot t % S),
//   * S^T of tile j + 1 (kQK) from K slot (j+1) % S,
//   * the softmax of tile j,
//   * O^T += V^T P^T of tile j - 1 (kPV) from V slot (j-1) % S,
//   * the O rescale of tile j (after the P V of tile j - 1),
// then waits for K tile j + 2 and V tile j (read by step j + 1) and syncs.
template <int D, bool kNeg, int kJ4, bool kQK, bool kPV, bool kMask, bool kLast = false>
__device__ __forceinline__ void step(WaveState<D>& w, uint32_t lds, int j, int N,
                                     float c_log2, int wave, int hh, bool first) {
  using G = FGeo<D>;
  constexpr int kPar = kJ4 & 1;
  constexpr uint32_t kTileB = G::kTile * 2;
  const uint32_t k_rd = lds + ((kJ4 + 1) % kSlots) * kTileB;
  const uint32_t v_rd = lds + (kSlots + (kJ4 + kSlots - 1) % kSlots) * kTileB;
  constexpr int kU = G::kUnits;
  constexpr int kAhead = 2;                  // LDS fragment reads run this many units ahead
  // The step's tile loads are issued between its products (after units
  // kDmaK and kDmaV), not in one burst at its start: measured faster.  Their
  // slots (K tile j, V tile j - 2) are not read in this step, and their order
  // among all loads, which the waits below count on, is unchanged.
  constexpr int kDmaK = kU / 4, kDmaV = (5 * kU) / 8;

  SoftmaxScratch sc;
  const int valid = N - j * kBc;             // keys of tile j that exist (mask)
  // fragments: K frag u and V^T frag u (u = s2 * kDB + db) of this step
  bf16x8 kf[kU], vf[kU];
#pragma unroll
  for (int u = 0; u < kAhead; ++u) {
    if (kQK) kf[u] = lds_k(k_rd, w.koff[u]);
    if (kPV) vf[u] = lds_vt(v_rd + (u / G::kDB) * 16 * D * 2, w.voff[u % G::kDB], hi_off<D>(w, u % G::kDB));
  }
  fence();
  constexpr int kSlotsUsed = (kQK ? 2 * kU : 0) + (kPV ? 2 * kU : 0);
  constexpr int kPerUnit = kSlotsUsed / kU;  // MFMA slots per unit
  constexpr TaskSplit<(kSlotsUsed > 0 ? kSlotsUsed : 1)> kSplit{};
  if (kSlotsUsed > 0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (u == kDmaK) dma_next<D>(w.dvoff, w.kp, w.kleft, w.dleft, N, lds + kJ4 * kTileB, wave);
      if (u == kDmaV)
        dma_next<D>(w.dvoff, w.vp, w.vleft, w.dleft, N,
                    lds + (kSlots + (kJ4 + kSlots - 2) % kSlots) * kTileB, wave);
      if (u + kAhead < kU) {
        if (kQK) kf[u + kAhead] = lds_k(k_rd, w.koff[u + kAhead]);
        if (kPV)
          vf[u + kAhead] = lds_vt(v_rd + ((u + kAhead) / G::kDB) * 16 * D * 2,
                                  w.voff[(u + kAhead) % G::kDB], hi_off<D>(w, (u + kAhead) % G::kDB));
      }
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const bool is_qk = mm < 2;
        if (is_qk && !kQK) continue;
        if (!is_qk && !kPV) continue;
        const int qb = mm & 1;
        const int slot = u * kPerUnit + ((kQK && !is_qk) ? 2 : 0) + qb;
        if (is_qk) {
          w.s[kPar ^ 1][qb] = mfma32x32x16(kf[u], w.qf[qb][u], u == 0 ? f32x16{} : w.s[kPar ^ 1][qb]);
        } else {
          const int s2 = u / G::kDB, db = u % G::kDB;
          mfma_oacc<kLast>(w.oacc[qb][db], vf[u], as_bf16x8(w.p[kPar ^ 1][qb][s2]));
        }
#pragma unroll
        for (int t = kSplit.b[slot]; t < kSplit.b[slot + 1]; ++t)
          softmax_task<D, kNeg, kMask, kPar>(t, w, sc, c_log2, valid, hh);
        fence();
      }
    }
  } else {
    dma_next<D>(w.dvoff, w.kp, w.kleft, w.dleft, N, lds + kJ4 * kTileB, wave);
    dma_next<D>(w.dvoff, w.vp, w.vleft, w.dleft, N,
                lds + (kSlots + (kJ4 + kSlots - 2) % kSlots) * kTileB, wave);
#pragma unroll
    for (int t = 0; t < kTasks; ++t) softmax_task<D, kNeg, kMask, kPar>(t, w, sc, c_log2, valid, hh);
  }
  // The weights and sums of this tile are consumed by the next step: make
  // them here, beside the products they overlap, not after the barrier.
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) asm volatile("" : "+v"(w.p[kPar][qb][s2]));
    asm volatile("" : "+v"(w.l[qb]), "+v"(w.m[qb]));
  }
  if (first) {
    // the first tile (alpha = 0 where the max moved): O starts here, not
    // live before this step, zero in AGPRs as a product of zeros with a
    // zero accumulator (the s_nop covers the zero operand just written)
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int db = 0; db < G::kDB; ++db) {
        const bf16x8 z = {};
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "=a"(w.oacc[qb][db]) : "v"(z));
      }
  } else if (sc.need) {
    oacc_settle(w.oacc);
    // one accumulator at a time through the vector ALU (16 VGPRs, not 128)
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int db = 0; db < G::kDB; ++db) {
        f32x16 t = w.oacc[qb][db];
        asm volatile("" : "+v"(t));
        t *= sc.alpha[qb];
        asm volatile("" : "+v"(t));
        w.oacc[qb][db] = t;
        asm volatile("" : "+a"(w.oacc[qb][db]));
      }
  }
  // K tile j+2 and V tile j (next step's reads) must have landed.  Loads
  // issue in the order K_0 .. K_{S-1}, V_0 .. V_{S-3} (prologue), then
  // K_{t+S}, V_{t+S-2} at step t (S = kSlots); the later of the two, V_j,
  // is followed by 2 (S - 2) tile loads once j >= S - 2, and by at least
  // S - 1 before that.
  if (j >= kSlots - 2)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * (kSlots - 2) * G::kDma) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((kSlots - 1) * G::kDma) : "memory");
}

// O^T += V^T P^T of the last tile (V slot kJ4), outside the pipeline.
template <int D, int kJ4>
__device__ __forceinline__ void pv_last(WaveState<D>& w, uint32_t lds) {
  using G = FGeo<D>;
  constexpr int kPar = kJ4 & 1;
  const uint32_t v_rd = lds + (kSlots + kJ4) * (G::kTile * 2);
#pragma unroll
  for (int u = 0; u < G::kUnits; ++u) {
    const int s2 = u / G::kDB, db = u % G::kDB;
    const bf16x8 vf = lds_vt(v_rd + s2 * 16 * D * 2, w.voff[db], hi_off<D>(w, db));
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
      mfma_oacc<true>(w.oacc[qb][db], vf, as_bf16x8(w.p[kPar][qb][s2]));
  }
}

template <int D, bool kNeg, int kJ4, bool kMask>
__device__ __forceinline__ void last_step(WaveState<D>& w, uint32_t lds, int j, int N,
                                          float c_log2, int wave, int hh, bool single) {
  if (single)
    step<D, kNeg, kJ4, false, false, kMask, true>(w, lds, j, N, c_log2, wave, hh, true);
  else
    step<D, kNeg, kJ4, false, true, kMask, true>(w, lds, j, N, c_log2, wave, hh, j == 0);
  pv_last<D, kJ4>(w, lds);
}

// Middle steps j0 .. j0 + kSlots - 1 (j0 % kSlots == 1), stopping before
// the last tile: every step's slots are compile-time constants.
template <int D, bool kNeg, size_t... I>
__device__ __forceinline__ void middle_round(WaveState<D>& w, uint32_t lds, int j0,
                                             int n_tiles, int N, float c_log2, int wave, int hh,
                                             std::index_sequence<I...>) {
  bool go = true;
  ((go = go && (j0 + (int)I < n_tiles - 1) &&
         (step<D, kNeg, (int)((I + 1) % kSlots), true, true, false>(w, lds, j0 + (int)I, N,
                                                                    c_log2, wave, hh, false),
          true)),
   ...);
}

// The last step of tile jl, its slot picked from jl % kSlots at run time.
template <int D, bool kNeg, bool kMask, size_t... I>
__device__ __forceinline__ void last_round(WaveState<D>& w, uint32_t lds, int jl, int N,
                                           float c_log2, int wave, int hh,
                                           std::index_sequence<I...>) {
  ((jl % kSlots == (int)I
        ? (last_step<D, kNeg, (int)I, kMask>(w, lds, jl, N, c_log2, wave, hh, false), 0)
        : 0),
   ...);
}

#if ATTN_ROWS64_SPLIT
// The split-KV form: the workgroup covers one of n_split contiguous key
// ranges of chunk_keys keys (whole tiles) and writes its partial result --
// O of its keys normalised by their own exp-sum, and their log-sum-exp --
// as fp32 to part_o / part_lse, rows of all heads numbered as in lse; the
// merge kernel combines the ranges.
template <int D, bool kNeg>
__global__ __launch_bounds__(kFThreads, 1)
void attn_fwd_bf16_rows64_split_kernel(const __bf16* __restrict__ q,
                                       const __bf16* __restrict__ k,
                                       const __bf16* __restrict__ v, int Hq, int Hkv, int N,
                                       float c_log2, int n_qtiles, uint32_t n_xcd, int n_split,
                                       int chunk_keys, int64_t n_rows, float* __restrict__ part_o,
                                       float* __restrict__ part_lse) {
#else
// rev_every: 0, or the workgroups one XCD runs at a time (one round); odd
// rounds then stream the keys in reverse order (N a multiple of kBc only).
template <int D, bool kNeg>
__global__ __launch_bounds__(kFThreads, 1)
void attn_fwd_bf16_rows64_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                          const __bf16* __restrict__ v, __bf16* __restrict__ o,
                          float* __restrict__ lse, int Hq, int Hkv, int N, float c_log2,
                          int n_qtiles, uint32_t n_xcd, uint32_t rev_every) {
#endif
  using G = FGeo<D>;
  // K slots then V slots, kBc x D bf16 each
  __shared__ __align__(16) __bf16 smem[2 * kSlots * G::kTile];
  const uint32_t lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) __bf16*)smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

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
  uint32_t rest = logical / (uint32_t)n_qtiles;
#if ATTN_ROWS64_SPLIT
  // the key range next: all query tiles of one range run side by side
  const int split = (int)(rest % (uint32_t)n_split);
  rest /= (uint32_t)n_split;
#endif
  const int kvh = (int)(rest % (uint32_t)Hkv);
  const int b = (int)(rest / (uint32_t)Hkv);

  const int n_qrows = (Hq / Hkv) * N;                                // rows of the group
  const int64_t head_q = ((int64_t)b * Hkv + kvh) * (int64_t)n_qrows; // its first row
  const int64_t head_kv = ((int64_t)b * Hkv + kvh) * (int64_t)N;
#if ATTN_ROWS64_SPLIT
  // this workgroup's keys: the range [k0, k0 + Nk) of its split
  const int k0 = split * chunk_keys;
  const int Nk = min(chunk_keys, N - k0);
  const __bf16* kh = k + (head_kv + k0) * D;
  const __bf16* vh = v + (head_kv + k0) * D;
#else
  const __bf16* kh = k + head_kv * D;
  const __bf16* vh = v + head_kv * D;
#endif
  const int n_tiles = (ATTN_KEYS + kBc - 1) / kBc;

  WaveState<D> w;
#if ATTN_ROWS64_SPLIT
  w.rev_last = 0;
#else
  // this workgroup's round on its XCD (workgroups are dealt round-robin)
  const bool stream_hints = rev_every != 0;
  w.rev_last = (stream_hints && (((blockIdx.x / n_xcd) / rev_every) & 1u) != 0)
                   ? (n_tiles - 1) * kBc : 0;
#endif
  // ---- Q^T fragments: lane holds d = 16 s + 8 hh .. +7 of its queries -----
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int qrow = qt * kFBr + wave * kFRows + qb * 32 + l32;
    const bool qvalid = qrow < n_qrows;
    const __bf16* qp = q + (head_q + (qvalid ? qrow : 0)) * D + 8 * hh;
#pragma unroll
    for (int st = 0; st < G::kKSteps; ++st) {
      // read once: a streaming load, so Q does not displace K/V lines from the L2
      u32x4 u = qvalid ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qp + 16 * st))
                       : u32x4{0u, 0u, 0u, 0u};
      w.qf[qb][st] = as_bf16x8(u);
    }
  }
  // direct loads: instruction i of this wave fills chunks slot .. slot + 63
  // of a tile; lane's chunk g = slot + lane holds logical chunk
  // (g % kCPR) ^ swz<D>(row) of row g / kCPR.
#pragma unroll
  for (int i = 0; i < G::kDma; ++i) {
    const int g = (wave * G::kDma + i) * kWave + lane;
    const int row = g / G::kCPR;
    const int c = (g % G::kCPR) ^ swz<D>(row);
    w.dvoff[i] = (row * D + c * 8) * 2;
  }
  // K operand: row l32, chunk 2 s + hh, swizzled by the row.
#pragma unroll
  for (int st = 0; st < G::kKSteps; ++st)
    w.koff[st] = (l32 * D + (((2 * st + hh) ^ swz<D>(l32)) * 8)) * 2;
  // V^T operand (transposing read): in each 16-lane group, lane i points at
  // key (i / 4) of a 4-key run and d columns 4 (i % 4) .. +3 of the group's
  // 16 columns; it receives key run 0..3 of column (group base + i).
  {
    const int li = lane & 15;
    const int dhalf = (lane >> 4) & 1;
    const int vrow = 4 * hh + (li >> 2);   // row within a 16-key step (plus 8 for slots 4..7)
#pragma unroll
    for (int db = 0; db < G::kDB; ++db) {
      const int dcol = db * 32 + dhalf * 16 + 4 * (li & 3);
      w.voff[db] = (vrow * D + (((dcol >> 3) ^ swz<D>(vrow)) * 8) + (dcol & 7)) * 2;
      if (D == 64) w.voff8[db] = ((vrow + 8) * D + (((dcol >> 3) ^ swz<D>(vrow + 8)) * 8) + (dcol & 7)) * 2;
    }
  }
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    w.m[qb] = -INFINITY;
    w.l[qb] = 0.0f;
  }

  // ---- prologue: K tiles 0 .. S-1 and V tiles 0 .. S-3 in flight; S of tile 0
  constexpr uint32_t kTileB = G::kTile * 2;
  {
    const bool rev = w.rev_last > 0;
    const int first = rev ? w.rev_last : 0;
    w.kp = reinterpret_cast<const char*>(kh + (int64_t)first * D);
    w.vp = reinterpret_cast<const char*>(vh + (int64_t)first * D);
    w.kleft = w.vleft = ATTN_KEYS - first;
    w.dleft = rev ? kBc : -kBc;
  }
#pragma unroll
  for (int t = 0; t < kSlots; ++t)
    dma_next<D>(w.dvoff, w.kp, w.kleft, w.dleft, ATTN_KEYS, lds + t * kTileB, wave);
#pragma unroll
  for (int t = 0; t < kSlots - 2; ++t)
    dma_next<D>(w.dvoff, w.vp, w.vleft, w.dleft, ATTN_KEYS, lds + (kSlots + t) * kTileB, wave);
  // K tiles 0 and 1 must have landed: S of tile 0 reads K slot 0 here and
  // step 0 reads K slot 1 (for S of tile 1) before its own wait; the other
  // 2 kSlots - 4 tiles may still be in flight
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((2 * kSlots - 4) * G::kDma) : "memory");
#pragma unroll
  for (int st = 0; st < G::kKSteps; ++st) {
    const bf16x8 kf = lds_k(lds, w.koff[st]);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
      w.s[0][qb] = mfma32x32x16(kf, w.qf[qb][st], st == 0 ? f32x16{} : w.s[0][qb]);
  }
  // every wave has read K slot 0 before step 0 reloads it
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  const bool tail = (ATTN_KEYS % kBc) != 0;
  if (n_tiles == 1) {
    if (tail) last_step<D, kNeg, 0, true>(w, lds, 0, ATTN_KEYS, c_log2, wave, hh, true);
    else last_step<D, kNeg, 0, false>(w, lds, 0, ATTN_KEYS, c_log2, wave, hh, true);
  } else {
    step<D, kNeg, 0, true, false, false>(w, lds, 0, ATTN_KEYS, c_log2, wave, hh, true);
    // middle steps 1 .. n_tiles - 2, unrolled by the ring size so every
    // slot index is a constant
    for (int j = 1; j < n_tiles - 1; j += kSlots)
      middle_round<D, kNeg>(w, lds, j, n_tiles, ATTN_KEYS, c_log2, wave, hh,
                            std::make_index_sequence<kSlots>{});
    const int jl = n_tiles - 1;
    oacc_settle(w.oacc);
    if (tail)
      last_round<D, kNeg, true>(w, lds, jl, ATTN_KEYS, c_log2, wave, hh, std::make_index_sequence<kSlots>{});
    else
      last_round<D, kNeg, false>(w, lds, jl, ATTN_KEYS, c_log2, wave, hh, std::make_index_sequence<kSlots>{});
  }
  // loads past the last tile may still be writing LDS: drain before exit
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#if !ATTN_ROWS64_SPLIT
  // the epilogue may stage O in the ring: every wave must be done reading it
  if (stream_hints) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#endif

  oacc_settle(w.oacc);
  // ---- epilogue: O = O~ / l, lse = (m + log2 l) ln 2 ------------------------
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int qrow = qt * kFBr + wave * kFRows + qb * 32 + l32;
    const float l_tot = xhalf_sum(w.l[qb]);
#if ATTN_ROWS64_SPLIT
    if (qrow < n_qrows) {
      // partial result of this key range: O / l in fp32 and its lse
      const float inv = 1.0f / l_tot;
      const int64_t prow = (int64_t)split * n_rows + head_q + qrow;
      float* orow = part_o + prow * D;
#pragma unroll
      for (int db = 0; db < G::kDB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f32x4 ov;
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = w.oacc[qb][db][4 * r + i] * inv;
          *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * r + 4 * hh) = ov;
        }
      if (hh == 0) part_lse[prow] = (w.m[qb] + log2_fast(l_tot)) * 0.69314718055994531f;
    }
#else
    const float inv = 1.0f / l_tot;
    if (stream_hints) {
      // O through LDS: the wave stages its block's 32 rows (rows of D bf16 +
      // 16 bytes, against bank conflicts), then every store writes whole
      // rows, non-temporal (partial-line stores left in the L2 would be
      // written back piecemeal)
      constexpr int kRowB = D * 2 + 16;
      const uint32_t stage = lds + (uint32_t)(wave * 32 * kRowB);
#pragma unroll
      for (int db = 0; db < G::kDB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u32x2 wv;
          wv[0] = pack_bf16x2(w.oacc[qb][db][4 * r + 0] * inv, w.oacc[qb][db][4 * r + 1] * inv);
          wv[1] = pack_bf16x2(w.oacc[qb][db][4 * r + 2] * inv, w.oacc[qb][db][4 * r + 3] * inv);
          *(lds_u32x2*)(uintptr_t)(stage + l32 * kRowB + (db * 32 + 8 * r + 4 * hh) * 2) = wv;
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's rows are staged
      constexpr int kChunks = D / 8;                        // 16-byte chunks per row
      constexpr int kRowsPer = kWave / kChunks;             // rows per store
#pragma unroll
      for (int i = 0; i < 32 / kRowsPer; ++i) {
        const int rr = i * kRowsPer + lane / kChunks;
        const int ch = lane % kChunks;
        const u32x4 v4 = *(const lds_u32x4*)(uintptr_t)(stage + rr * kRowB + ch * 16);
        const int row = qt * kFBr + wave * kFRows + qb * 32 + rr;
        if (row < n_qrows)
          __builtin_nontemporal_store(v4, reinterpret_cast<u32x4*>(o + (head_q + row) * D + ch * 8));
      }
      // the next block's staging writes must not pass these reads
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    } else if (qrow < n_qrows) {
      __bf16* orow = o + (head_q + qrow) * D;
#pragma unroll
      for (int db = 0; db < G::kDB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u32x2 wv;
          wv[0] = pack_bf16x2(w.oacc[qb][db][4 * r + 0] * inv, w.oacc[qb][db][4 * r + 1] * inv);
          wv[1] = pack_bf16x2(w.oacc[qb][db][4 * r + 2] * inv, w.oacc[qb][db][4 * r + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * r + 4 * hh) = wv;
        }
    }
    if (qrow < n_qrows && hh == 0)
      lse[head_q + qrow] = (w.m[qb] + log2_fast(l_tot)) * 0.69314718055994531f;
#endif
  }
}


}  // namespace
}  // namespace attn
