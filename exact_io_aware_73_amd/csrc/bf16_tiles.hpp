// bf16_tiles.hpp -- K / V tile staging for the bf16 MFMA kernels.
//
// Tile geometry shared by the fused forward and the materialising path's
// P V kernel: a workgroup of 4 waves stages kBc keys of K (row-major) and V
// (transposed, keys fastest) per stage.  Row strides are padded so that
//   * the K rows read as MFMA A operands (16 bytes per lane, 32 keys) and
//   * the V^T rows read as MFMA operands (8 bytes per lane, 32 d values)
// fall on distinct LDS banks, and the staging map below keeps the
// transposing writes conflict-free as well.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace attn {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;   // query rows per workgroup

template <int D>
struct Geo {
  static constexpr int kBc = (D == 128) ? 64 : 128;   // keys per tile
  static constexpr int kKB = kBc / 32;                // 32-key blocks per tile
  static constexpr int kKSteps = D / 16;              // MFMA k-steps over d
  static constexpr int kDB = D / 32;                  // 32-wide d blocks
  static constexpr int kKStr = D + 8;                 // LDS K row stride (bf16)
  static constexpr int kVStr = kBc + 4;               // LDS V^T row stride (bf16)
  static constexpr int kKElems = kBc * kKStr;
  static constexpr int kVElems = D * kVStr;
  static constexpr int kStage = kKElems + kVElems;    // bf16 elements per stage
  static constexpr int kLdsBytes = 2 * kStage * 2;
  static constexpr int kDG = D / 8;                   // 16-byte chunks per row
  static constexpr int kKChunks = kBc * D / 8 / kThreads;  // K chunks per thread
  static_assert(kBc * D / 8 == 4 * kThreads, "staging map assumes 4 chunks per thread");
  static_assert((kBc / 4) * kDG == kThreads, "V^T staging: one 4x8 block per thread");
};

struct Regs {
  u32x4 k[4];
  u32x4 v[4];
};

// V staging map: a thread owns 4 consecutive keys x 8 consecutive d.  Thread
// bits 0..2 give the low bits of its 4-key group and the next log2(kDG) bits
// its d group, so the 16 lanes that an LDS write cycle serves cover 8 key
// groups x 2 d groups and hit 16 distinct 8-byte banks.
template <int D>
__device__ __forceinline__ int v_key_group(int tid) {
  return (tid & 7) | ((tid >> (3 + __builtin_ctz(Geo<D>::kDG))) << 3);
}
template <int D>
__device__ __forceinline__ int v_d_group(int tid) {
  return (tid >> 3) & (Geo<D>::kDG - 1);
}

// Global -> registers, K tile starting at key j0 (4 x 16 bytes per thread,
// consecutive threads on consecutive 16-byte chunks).  Rows at or beyond N
// read as zeros; nothing is read out of bounds.
template <int D>
__device__ __forceinline__ void load_k_tile(Regs& r, const __bf16* __restrict__ kh, int j0, int N,
                                            int tid) {
  using G = Geo<D>;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + i * kThreads;
    const int row = c / G::kDG;
    const int col = (c % G::kDG) * 8;
    const int key = j0 + row;
    r.k[i] = key < N ? *reinterpret_cast<const u32x4*>(kh + (int64_t)key * D + col)
                     : u32x4{0u, 0u, 0u, 0u};
  }
}

// Global -> registers, V tile starting at key j0 (the thread's 4 key rows).
template <int D>
__device__ __forceinline__ void load_v_tile(Regs& r, const __bf16* __restrict__ vh, int j0, int N,
                                            int tid) {
  const int kg = v_key_group<D>(tid);
  const int dg = v_d_group<D>(tid);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int key = j0 + kg * 4 + rr;
    r.v[rr] = key < N ? *reinterpret_cast<const u32x4*>(vh + (int64_t)key * D + dg * 8)
                      : u32x4{0u, 0u, 0u, 0u};
  }
}

// Registers -> LDS, K row-major [kBc][kKStr].
template <int D>
__device__ __forceinline__ void store_k_tile(const Regs& r, __bf16* __restrict__ ks, int tid) {
  using G = Geo<D>;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + i * kThreads;
    const int row = c / G::kDG;
    const int col = (c % G::kDG) * 8;
    *reinterpret_cast<u32x4*>(ks + row * G::kKStr + col) = r.k[i];
  }
}

// Registers -> LDS, V transposed [D][kVStr]: a 4 x 8 register transpose
// (v_perm_b32 on 16-bit halves), then eight 8-byte writes.
template <int D>
__device__ __forceinline__ void store_v_tile(const Regs& r, __bf16* __restrict__ vts, int tid) {
  using G = Geo<D>;
  const int kg = v_key_group<D>(tid);
  const int dg = v_d_group<D>(tid);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // word w of each key row holds d = dg*8 + 2w (low half) and +1 (high half)
    const uint32_t a0 = r.v[0][w], a1 = r.v[1][w], a2 = r.v[2][w], a3 = r.v[3][w];
    u32x2 lo, hi;
    lo[0] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);   // keys 0,1 of the even d
    lo[1] = __builtin_amdgcn_perm(a3, a2, 0x05040100u);   // keys 2,3 of the even d
    hi[0] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);   // keys 0,1 of the odd d
    hi[1] = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
    const int d = dg * 8 + 2 * w;
    *reinterpret_cast<u32x2*>(vts + d * G::kVStr + kg * 4) = lo;
    *reinterpret_cast<u32x2*>(vts + (d + 1) * G::kVStr + kg * 4) = hi;
  }
}

template <int D>
__device__ __forceinline__ void load_tile(Regs& r, const __bf16* __restrict__ kh,
                                          const __bf16* __restrict__ vh, int j0, int N, int tid) {
  load_k_tile<D>(r, kh, j0, N, tid);
  load_v_tile<D>(r, vh, j0, N, tid);
}

template <int D>
__device__ __forceinline__ void store_tile(const Regs& r, __bf16* __restrict__ ks,
                                           __bf16* __restrict__ vts, int tid) {
  store_k_tile<D>(r, ks, tid);
  store_v_tile<D>(r, vts, tid);
}

}  // namespace attn
