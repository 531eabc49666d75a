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
  int n_cu = 0;        // compute units of the device
  int l2_bytes = 0;    // L2 cache of one XCD, bytes
  // split-KV path only: the key ranges, their length (whole tiles) and the
  // fp32 partial results [n_split][B*Hq*N][d] and [n_split][B*Hq*N]
  int n_split = 1;
  int chunk_keys = 0;
  float* part_o = nullptr;
  float* part_lse = nullptr;
  // 8-bit path only: the V scale (q, k, v are E4M3 codes; v is V^T, [B,Hkv,d,Np];
  // scale already holds scale * q_scale * k_scale)
  float v_scale = 1.0f;
  hipStream_t stream;
};

// workgroup counts (for the launch-size check)
uint64_t fwd_bf16_rows32_grid(int B, int Hq, int Hkv, int N);
uint64_t fwd_bf16_rows64_grid(int B, int Hq, int Hkv, int N);
uint64_t fwd_f32_grid(int B, int Hq, int N);

// Fused bf16 forward, two kernel designs:
//   rows32 -- one 32-row query block per wave, 128 query rows per
//             workgroup; four workgroups per CU at head dim 64, two at 128;
//   rows64 -- two 32-row query blocks per wave sharing every K / V fragment
//             read from LDS, software-pipelined across key tiles, 256 query
//             rows per workgroup, one workgroup per CU (head dim 128).
// Head dim 128 takes rows64 where the keys are not short (N >= 1024) and its
// grid has at least one workgroup per CU; elsewhere rows32, whose smaller
// workgroups spread a small grid over every CU and hide the per-workgroup
// start and end behind a second workgroup (measured, rows64 against rows32
// with a full grid: N = 4096 +5 ... +6 %, 2048 +5 %, 1024 +2 %, 512 -6 %,
// 256 -10 %; one head of 32768 rows, 128 workgroups, rows32 +39 %).  n_cu is
// the device's compute-unit count (read from the HIP runtime once per
// device).
hipError_t launch_fwd_bf16_rows32(const FwdArgs& a);
hipError_t launch_fwd_bf16_rows64(const FwdArgs& a);
inline bool fwd_bf16_use_rows64(int B, int Hq, int Hkv, int N, int d, int n_cu) {
  return d == 128 && N >= 1024 && fwd_bf16_rows64_grid(B, Hq, Hkv, N) >= (uint64_t)n_cu;
}
hipError_t launch_fwd_f32(const FwdArgs& a);

// 8-bit (OCP E4M3) forward on the FP8 MFMA; V^T rows of Np = fp8_padded_keys(N) bytes.
int fp8_padded_keys(int N);
uint64_t fwd_fp8_grid(int B, int Hq, int Hkv, int N);
hipError_t launch_fwd_fp8(const FwdArgs& a);

// Backward (bf16): D = rowsum(dO * O) into dvec (fp32, B*Hq*N), then dK/dV
// and dQ, recomputing S and P from q, k and lse.  a.o is the forward's O.
struct BwdArgs {
  const void* dout;   // dL/dO, like q
  void* dq;           // like q
  void* dk;           // like k
  void* dv;           // like v
  float* dvec;        // workspace: B*Hq*N floats
};
uint64_t bwd_grid(int B, int Hq, int Hkv, int N);
hipError_t launch_bwd_bf16(const FwdArgs& a, const BwdArgs& g);

// Split-KV forward (bf16): the rows64 kernel over key ranges of
// split_chunk_keys(N, n_split) keys into part_o / part_lse, then the merge
// of the ranges into o / lse.  The number of non-empty ranges is
// ceil(N / chunk_keys), which may be below the requested n_split.
uint64_t split_chunk_keys(int N, int n_split);
hipError_t launch_fwd_bf16_split(const FwdArgs& a);
hipError_t launch_split_merge_bf16(const FwdArgs& a);
hipError_t launch_materialized_bf16(const FwdArgs& a);
hipError_t launch_materialized_f32(const FwdArgs& a);

}  // namespace attn
