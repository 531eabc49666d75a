// kernels.hpp -- host-side launchers of the HIP kernels in libattn.so.
// Arguments are validated by the C-ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* s;    // materialising path only: [B,Hq,N,N] fp32 scores
  void* p;     // materialising path only: [B,Hq,N,N] weights (I/O dtype)
  int B, Hq, Hkv, N, d;
  float scale;
  int n_xcd;
  hipStream_t stream;
};

// workgroup counts (for the launch-size check)
uint64_t fwd_bf16_grid(int B, int Hq, int N);
uint64_t fwd_f32_grid(int B, int Hq, int N);

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_materialized_bf16(const FwdArgs& a);
hipError_t launch_materialized_f32(const FwdArgs& a);

}  // namespace attn
