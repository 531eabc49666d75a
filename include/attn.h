/*
 * attn.h -- C ABI of libattn.so: exact scaled-dot-product attention forward
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation (every entry point below computes it):
 *
 *   For each batch b in [0,B) and query head h in [0,Hq), with the shared
 *   key/value head kv = h / (Hq / Hkv) (contiguous groups of query heads
 *   share one K/V head: grouped-query attention, "efficient attention"
 *   course chapter (deeplearning.wizardwu.top), class 3 and its methods
 *   table), and each query row i:
 *
 *     S[i,j]     = scale * sum_c q[b,h,i,c] * k[b,kv,j,c]
 *     O[b,h,i,:] = sum_j softmax_j(S[i,:]) * v[b,kv,j,:]
 *     lse[b,h,i] = ln sum_j exp(S[i,j])
 *
 *   i.e. O = softmax(Q K^T * scale) V per head (aiknowledge.cn
 *   "1.1 注意力计算的计算与显存瓶颈", section 1.1.1; blog
 *   "attention 的显存线性化", section 一), with no mask and no dropout.
 *   `scale` is usually 1/sqrt(d); any finite value is accepted.
 *
 * Layout: row-major, contiguous, head dimension fastest.
 *   q, o : [B, Hq,  N, d]
 *   k, v : [B, Hkv, N, d]
 *   lse  : [B, Hq,  N]      float32, natural logarithm
 *   s, p : [B, Hq,  N, N]   (materialising entry points only)
 *
 * Pointers: every array pointer is a DEVICE pointer, allocated and owned by
 * the caller.  The library allocates no device memory and keeps no state
 * between calls other than immutable device facts: the compute-unit and
 * XCD counts of each device, read from the HIP runtime once per device
 * (thread-safe, on the first call that launches work there).  Outputs
 * (o, lse, s, p) must not overlap the inputs or each other.
 *
 * Device: work runs on the calling thread's current HIP device, which must
 * be the device that holds the pointers and owns `stream`.
 *
 * Stream: `stream` is a hipStream_t passed as void*; NULL means the null
 * stream.  Work is enqueued and the call returns without synchronising.
 *
 * Errors: every argument is checked before any HIP call; a failed check
 * returns its attn_status_t code and enqueues nothing.  An error reported by
 * the HIP runtime (a launch, or the device query) returns ATTN_ERR_HIP.  No
 * entry point prints, aborts or lets an exception escape.  attn_strerror()
 * names a code.
 *
 * Sizes: B, Hq, Hkv, N >= 1; Hq % Hkv == 0; d in {64, 128}.  Element
 * offsets are computed in 64 bits; B*Hkv*ceil((Hq/Hkv)*N/128) workgroups
 * (the query tiles run over the adjacent rows of the heads that share a
 * K/V head) must fit the launch grid (< 2^31 / 256 workgroups).
 */
#ifndef ATTN_H_
#define ATTN_H_

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define ATTN_API __attribute__((visibility("default")))
#else
#define ATTN_API
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,     /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,    /* B, Hq, Hkv or N < 1, or the problem is too large */
  ATTN_ERR_GQA = 3,      /* Hq is not a multiple of Hkv */
  ATTN_ERR_HEADDIM = 4,  /* d is not 64 or 128 */
  ATTN_ERR_SCALE = 5,    /* scale is NaN or infinite */
  ATTN_ERR_ALIGN = 6,    /* q/k/v/o/s/p not 16-byte aligned, or lse not 4-byte aligned */
  ATTN_ERR_HIP = 7,      /* the HIP runtime reported an error (a launch, or a device query) */
  ATTN_ERR_ALIAS = 8,    /* an output overlaps an input or another output */
  ATTN_ERR_SPLIT = 9,    /* n_split outside [1, ATTN_MAX_SPLIT] */
  ATTN_ERR_WORKSPACE = 10, /* workspace NULL, misaligned or smaller than required */
  ATTN_ERR_SCRATCH = 11  /* more rows than the fixed scratch buffer of attn_bwd_noalloc holds */
} attn_status_t;

/* Largest number of key ranges the split-KV entry point accepts. */
#define ATTN_MAX_SPLIT 64

/*
 * attn_fwd -- fused tiled forward, bfloat16 I/O, float32 accumulation.
 *
 * The IO-aware method: the query rows of each head are split into tiles and
 * every tile streams all key/value tiles through on-chip memory, keeping a
 * running row maximum m and exp-sum l and rescaling earlier partial sums by
 * exp(m_old - m_new) when m grows (blog "attention 的显存线性化", section 三;
 * "efficient attention" chapter, online-softmax paragraph).  S and P never
 * reach device memory; O / l and lse are written once (aiknowledge.cn
 * "3.1 性能模型：用 Roofline 与算术强度算清为什么快", section 3.1.3).
 *
 * q, k, v, o: bf16 (__bf16 / uint16 bit patterns).  lse: float32.
 * Deterministic: the same inputs give bit-identical outputs.
 */
ATTN_API int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int N, int d, float scale, void* stream);

/*
 * attn_fwd_f32 -- the same fused tiled forward with float32 I/O and float32
 * arithmetic throughout (no reduced-precision products).
 */
ATTN_API int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int Hq, int Hkv, int N, int d, float scale, void* stream);

/*
 * attn_fwd_materialized -- the "standard attention" the pages compare
 * against (aiknowledge.cn "1.1 ...", sections 1.1.1 and 1.1.3): three
 * kernels on `stream`, each a full device-memory round trip of an [N, N]
 * matrix per head:
 *   1. S = scale * Q K^T        written to s   (float32, [B,Hq,N,N])
 *   2. P = row softmax of S     written to p   (bf16, [B,Hq,N,N]), and lse
 *   3. O = P V                  written to o   (bf16)
 * q, k, v, o, p: bf16.  s, lse: float32.  The caller sizes s and p
 * (4 and 2 bytes per element) and may read them afterwards.
 */
ATTN_API int attn_fwd_materialized(const void* q, const void* k, const void* v, void* o,
                                   float* lse, float* s, void* p,
                                   int B, int Hq, int Hkv, int N, int d, float scale,
                                   void* stream);

/*
 * attn_fwd_materialized_f32 -- the materialising path with float32 I/O:
 * q, k, v, o, s, p and lse all float32.
 */
ATTN_API int attn_fwd_materialized_f32(const float* q, const float* k, const float* v, float* o,
                                       float* lse, float* s, float* p,
                                       int B, int Hq, int Hkv, int N, int d, float scale,
                                       void* stream);

/*
 * attn_fwd_fp8 -- the fused tiled forward with 8-bit floating-point inputs
 * on the FP8 matrix cores (the pages list FP8 among the third FlashAttention
 * version's features without its arithmetic: blog "attention 的显存线性化",
 * section 五).
 *
 * q8  : [B, Hq,  N,  d]  OCP 8-bit floating point E4M3 codes (1 sign, 4
 *                        exponent bits with bias 7, 3 mantissa bits; no
 *                        infinities; 0x7F / 0xFF are NaN), one byte each
 * k8  : [B, Hkv, N,  d]  E4M3
 * vt8 : [B, Hkv, d, Np]  E4M3, V TRANSPOSED (key index fastest), rows padded
 *                        to Np = N rounded up to a multiple of 16 keys; the
 *                        padding bytes are ignored (they may hold anything)
 * o   : [B, Hq,  N,  d]  bf16;   lse : [B, Hq, N] float32, natural log
 * The values are q = q_scale * q8, k = k_scale * k8, v = v_scale * v8; the
 * result is attention of those values with `scale` as in attn_fwd.
 *
 * Accuracy contract: the scores are the exact 8-bit products summed by
 * the matrix core into fp32, within 2^-14 * |scale| * sum_c |q_c k_c| of
 * exact; lse uses the unrounded weights, so its error is that of the
 * scores.  The one lossy step: each softmax weight p = exp(S - m) -- m a
 * running row maximum, at most 2 (log2 units) below the row's true maximum
 * when the largest weights are met -- is scaled by 2^6 and rounded to E4M3
 * before the PV product (relative error <= 2^-4; absolute error <= 2^-16
 * of the row's largest weight); the exp-sum uses the unrounded weights.
 * Hence per element |O - O_exact| <= sum_j (2^-4 w_j + 2^-16 max_k w_k)
 * |v_jc|, plus the score error's effect, fp32 and the bf16 output
 * rounding, with w the exact softmax weights.
 *
 * Pointers: q8, k8, vt8, o 16-byte aligned, lse 4-byte aligned; outputs
 * must not overlap the inputs or each other.  q_scale, k_scale, v_scale and
 * scale * q_scale * k_scale must be finite (ATTN_ERR_SCALE).  d in {64, 128};
 * d * Np must be below 2^31.  Deterministic.
 */
ATTN_API int attn_fwd_fp8(const void* q8, const void* k8, const void* vt8, void* o, float* lse,
                          float q_scale, float k_scale, float v_scale, int B, int Hq, int Hkv,
                          int N, int d, float scale, void* stream);

/*
 * attn_fwd_split -- the fused forward with every head's keys cut into up to
 * n_split contiguous ranges of whole 32-key tiles, each range handled by its
 * own workgroups (for heads too few or too long to fill the GPU: one head of
 * 32768 rows gives 128 workgroups for 256 compute units).  Each range
 * writes its partial result -- O of its keys normalised by their own
 * exp-sum, and the log-sum-exp lse_r of its scores -- to the workspace; a
 * second kernel merges the ranges of every row by the online-softmax
 * rescale rule (blog "attention 的显存线性化", section 三):
 *   lse = ln sum_r exp(lse_r),   O = sum_r exp(lse_r - lse) * O_r.
 * Exact up to rounding, like attn_fwd; deterministic.
 *
 * bf16 q, k, v, o; float32 lse; same layouts as attn_fwd.  n_split in
 * [1, ATTN_MAX_SPLIT]; ranges hold ceil(ceil(N/32) / n_split) tiles, so
 * fewer than n_split ranges run when N is short.
 *
 * workspace: a DEVICE buffer owned by the caller, 16-byte aligned, of at
 * least attn_fwd_split_workspace_bytes(B, Hq, N, d, n_split) bytes; its
 * contents on entry do not matter and on return are unspecified.  It must
 * not overlap the inputs or outputs.  Two calls that share a workspace must
 * be ordered (same stream).
 */
ATTN_API int attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                            void* workspace, unsigned long long workspace_bytes, int n_split,
                            int B, int Hq, int Hkv, int N, int d, float scale, void* stream);

/*
 * attn_fwd_split_workspace_bytes -- workspace attn_fwd_split needs:
 * n_split * B * Hq * N * (d + 1) * 4 bytes (fp32 partial O and lse per
 * range and row).  0 for arguments attn_fwd_split would reject.
 */
ATTN_API unsigned long long attn_fwd_split_workspace_bytes(int B, int Hq, int N, int d,
                                                           int n_split);

/*
 * attn_bwd -- gradients of attn_fwd (bfloat16 I/O, float32 accumulation):
 * given q, k, v, the forward's o and lse, and dout = dL/dO, writes
 *   dq = dL/dQ, dk = dL/dK, dv = dL/dV
 * (a K/V head's gradient sums over the query heads that share it).  The
 * [N, N] matrices are recomputed block by block from q, k and lse, never
 * stored (blog "attention 的显存线性化", section 五; "efficient attention"
 * chapter, online-softmax section: recomputation in the backward pass).
 *
 * q, o, dout, dq: [B, Hq, N, d] bf16; k, v, dk, dv: [B, Hkv, N, d] bf16;
 * lse: [B, Hq, N] float32 from attn_fwd with the same inputs and scale.
 * workspace: a DEVICE buffer owned by the caller, 16-byte aligned, of at
 * least attn_bwd_workspace_bytes(B, Hq, N) bytes (the row sums of dO * O);
 * contents on entry do not matter.  Outputs and workspace must not overlap
 * the inputs or each other.  Deterministic (no atomic accumulation).
 */
ATTN_API int attn_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, unsigned long long workspace_bytes,
                      int B, int Hq, int Hkv, int N, int d, float scale, void* stream);

/* attn_bwd_workspace_bytes -- B * Hq * N * 4; 0 for B, Hq or N < 1. */
ATTN_API unsigned long long attn_bwd_workspace_bytes(int B, int Hq, int N);

/*
 * attn_bwd_noalloc -- attn_bwd without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving or training loops, harnesses that forbid allocation).  The same
 * kernels and results as attn_bwd; the per-row dot products go to a fixed
 * scratch buffer inside the library (16 MiB of device memory per device,
 * held until the process ends), so this call allocates nothing.
 *
 * Limit: B * Hq * N <= attn_bwd_noalloc_max_rows() (4194304 rows), else
 * ATTN_ERR_SCRATCH before any HIP call.  Every call on one device shares that
 * device's buffer: two calls that may run at the same time on one device
 * (different streams, or different threads without ordering) race and give
 * wrong gradients; order them on one stream.  Arguments, layouts and the
 * other errors as attn_bwd.
 */
ATTN_API int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              int B, int Hq, int Hkv, int N, int d, float scale, void* stream);

/* attn_bwd_noalloc_max_rows -- the largest B * Hq * N attn_bwd_noalloc accepts. */
ATTN_API unsigned long long attn_bwd_noalloc_max_rows(void);

/*
 * attn_device_info -- the device facts the launches use, for the calling
 * thread's current device: the number of compute units (the fused bf16
 * forward picks its kernel by it), of XCDs, the dies with their own L2 cache
 * over which workgroups are dealt round-robin (the launch order maps the
 * workgroups of one K/V head onto one XCD by it), and the L2 bytes the HIP
 * runtime reports (one XCD's; the head dim 128 kernel streams the keys of
 * alternate rounds of workgroups in reverse where a K/V head fits it).  Read
 * from the HIP runtime once per device and cached.  n_cu, n_xcd, l2_bytes:
 * host pointers, any may be NULL.  ATTN_ERR_HIP when the runtime cannot
 * report them.
 */
ATTN_API int attn_device_info(int* n_cu, int* n_xcd, int* l2_bytes);

/* Fused bf16 forward kernels (the value attn_fwd_plan writes). */
#define ATTN_KERNEL_ROWS32 1  /* 128 query rows per workgroup, one 32-row block per wave */
#define ATTN_KERNEL_ROWS64 2  /* 256 query rows per workgroup, two 32-row blocks per wave */

/*
 * attn_fwd_plan -- which kernel attn_fwd launches for these sizes on the
 * calling thread's current device: ATTN_KERNEL_ROWS64 for head dim 128 with
 * N >= 1024 and at least one 256-row workgroup per compute unit, else
 * ATTN_KERNEL_ROWS32.  The same argument checks as attn_fwd (pointers
 * aside); *kernel (host pointer, not NULL) is written only on ATTN_OK.
 */
ATTN_API int attn_fwd_plan(int B, int Hq, int Hkv, int N, int d, int* kernel);

/* attn_strerror -- a static, NUL-terminated description of a status code. */
ATTN_API const char* attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
