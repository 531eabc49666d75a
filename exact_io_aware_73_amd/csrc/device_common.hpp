// device_common.hpp -- small gfx950 device helpers shared by the HIP kernels
// of libattn.so (MFMA operand types, LDS/global vector access, launch-order
// remapping).  Device code only; written for CDNA4 (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16) on the matrix cores.
// Operand layout (lane l, half h = l / 32):
//   A: lane l holds row l % 32 and eight k values of group h;
//   B: lane l holds column l % 32 and the same eight k values of group h;
//   D: element 4*r + t of lane l is D[8*r + 4*h + t][l % 32].
// Both operands index k through the same (h, element) slot, so any fixed
// assignment of logical k to slots gives the same contraction.
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

// Round two floats to bf16 (round to nearest even) and pack them, first in
// the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ float exp2_fast(float x) {
  // v_exp_f32: 2^x; exp2(-inf) = 0.
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float log2_fast(float x) {
  return __builtin_amdgcn_logf(x);   // v_log_f32: log2(x)
}

// Workgroups are dispatched round-robin over the chip's XCDs (each with its
// own L2): physical id p runs on XCD p % n_xcd.  This maps p to a logical id
// so that every XCD receives one contiguous range of logical ids, in order;
// work items that share data (same K/V head) are numbered consecutively and
// so share an L2.  A bijection on [0, grid) for any grid size.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t p, uint32_t grid, uint32_t n_xcd) {
  const uint32_t xcd = p % n_xcd;
  const uint32_t slot = p / n_xcd;
  const uint32_t base = grid / n_xcd;
  const uint32_t extra = grid % n_xcd;
  return xcd * base + (xcd < extra ? xcd : extra) + slot;
}

}  // namespace attn
