"""Seeded synthetic inputs for exact attention forward.

This module holds the workload shapes and the seeded input generators, and
nothing of the attention arithmetic itself.  Both the CPU oracle's tests and
the GPU path's tests / benchmark draw their inputs from here, so the two
sides always see bit-identical tensors.

Inputs are i.i.d. standard normal, drawn on the CPU with a seeded
``torch.Generator`` in float32 and then rounded to the I/O dtype (round to
nearest even), so any host reproduces them exactly.  The pages measure only
one real workload (GPT-2-medium attention: n = 1024, d = 64, 16 heads,
batch 64; the "efficient attention" chapter, Dao et al. 2022 Fig. 2 table);
the shapes below stand in for it and for the long-sequence cases the pages
discuss, with synthetic values instead of a trained model's activations.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str            # "bf16" or "f32": the I/O element type
    seed: int             # base seed: +0 Q, +1 K, +2 V, +3 outlier rows
    k_outlier_frac: float = 0.0   # fraction of K rows (per (b, kv head)) scaled
    k_outlier_scale: float = 1.0  # by this power of two (exact in bf16)
    description: str = ""
    materialized: bool = True     # also time the S/P-materialising comparison path

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def shapes(self):
        return ((self.B, self.Hq, self.N, self.d),
                (self.B, self.Hkv, self.N, self.d))


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_n256_d64_f32", 1, 1, 1, 256, 64, "f32", 1000,
                 description="single head, fp32 I/O, small enough for the oracle in seconds"),
        Workload("gpt2_medium_b64_h16_n1024_d64", 64, 16, 16, 1024, 64, "bf16", 2000,
                 description="GPT-2-medium-shaped attention forward"),
        Workload("long_b4_h32_n4096_d128", 4, 32, 32, 4096, 128, "bf16", 3000,
                 description="long-sequence attention forward (also run materialized)"),
        Workload("gqa_b2_hq32_hkv8_n8192_d128", 2, 32, 8, 8192, 128, "bf16", 4000,
                 description="grouped-query attention, 4 query heads per K/V head"),
        Workload("gqa_b2_hq32_hkv8_n8192_d128_kscaled", 2, 32, 8, 8192, 128, "bf16", 4000,
                 k_outlier_frac=0.01, k_outlier_scale=8.0,
                 description="as above, 1% of K rows scaled by 8 to stress the running-max rescale"),
        Workload("long_context_b1_h8_n32768_d128", 1, 8, 8, 32768, 128, "bf16", 5000,
                 description="long-context attention forward; S+P would be 6.4 GB per head "
                             "(fp32 S, bf16 P), so only the tiled path runs",
                 materialized=False),
        Workload("one_head_b1_h1_n32768_d128", 1, 1, 1, 32768, 128, "bf16", 6000,
                 description="one long head: 128 query tiles of 256 rows for 256 compute "
                             "units, the case the split-KV path is for"),
        Workload("gqa_short_b64_hq32_hkv4_n200_d128", 64, 32, 4, 200, 128, "bf16", 7000,
                 description="grouped-query attention on short sequences, 8 query heads "
                             "per K/V head: heads shorter than a query tile"),
    ]
}

# The headline benchmark workload: the largest single-GPU configuration, at
# the long sequence lengths where the pages place the method's gain.
DEFAULT_BENCH = "long_context_b1_h8_n32768_d128"

# The sequence-length sweep ("3.1 性能模型：用 Roofline 与算术强度算清为什么快",
# section 3.1.5: every variable fixed but the sequence length, both arms
# measured at each length): the long_b4 configuration (B = 4, 32 heads,
# d = 128, bf16) at N = 512 ... 16384.  The comparison arm runs where its S
# and P fit (N <= 8192: 51.5 GB); at N = 16384 they would take 206 GB.
SWEEP_N = (512, 1024, 2048, 4096, 8192, 16384)
SWEEP = {
    w.name: w
    for w in [
        Workload(f"sweep_b4_h32_n{n}_d128", 4, 32, 32, n, 128, "bf16", 8000 + n,
                 description=f"sequence-length sweep at B = 4, 32 heads, d = 128: N = {n}",
                 materialized=n <= 8192)
        for n in SWEEP_N
    ]
}

# Every name bench.py accepts.
ALL = {**WORKLOADS, **SWEEP}


def _randn(shape, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def outlier_rows(N: int, frac: float, seed: int, n_slices: int) -> list[torch.Tensor]:
    """Row indices, per (b, kv head) slice, of the K rows to scale.

    round(frac * N) distinct rows per slice, drawn without replacement by a
    seeded permutation, one permutation per slice in (b, kv head) order.
    """
    count = int(round(frac * N))
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return [torch.randperm(N, generator=g)[:count] for _ in range(n_slices)]


def make_inputs(w: Workload, *, B=None, Hq=None, Hkv=None, N=None, d=None,
                dtype=None, seed=None):
    """Seeded CPU tensors (q, k, v) for workload ``w`` (fields may be overridden).

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d]; contiguous, in the I/O dtype.
    """
    B = w.B if B is None else B
    Hq = w.Hq if Hq is None else Hq
    Hkv = w.Hkv if Hkv is None else Hkv
    N = w.N if N is None else N
    d = w.d if d is None else d
    tdt = w.torch_dtype if dtype is None else dtype
    seed = w.seed if seed is None else seed
    q = _randn((B, Hq, N, d), seed + 0).to(tdt)
    k = _randn((B, Hkv, N, d), seed + 1).to(tdt)
    v = _randn((B, Hkv, N, d), seed + 2).to(tdt)
    if w.k_outlier_frac > 0.0:
        rows = outlier_rows(N, w.k_outlier_frac, seed + 3, B * Hkv)
        kf = k.view(B * Hkv, N, d)
        for s, idx in enumerate(rows):
            # a power-of-two factor: exact in bf16 and fp32
            kf[s, idx, :] = kf[s, idx, :] * w.k_outlier_scale
    return q.contiguous(), k.contiguous(), v.contiguous()


def random_inputs(B, Hq, Hkv, N, d, dtype: torch.dtype, seed: int, std: float = 1.0):
    """Seeded i.i.d. normal (q, k, v) of an arbitrary shape (for edge-case tests)."""
    q = (_randn((B, Hq, N, d), seed + 0) * std).to(dtype).contiguous()
    k = (_randn((B, Hkv, N, d), seed + 1) * std).to(dtype).contiguous()
    v = (_randn((B, Hkv, N, d), seed + 2) * std).to(dtype).contiguous()
    return q, k, v


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a CPU/GPU tensor (bf16 or fp32) to a float64 NumPy array."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


# ---------------------------------------------------------------------------
# 8-bit inputs (OCP E4M3 codes, one scale per tensor) for the FP8 entry point

def _e4m3_codes(x: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even E4M3 codes of x (|x| must stay within 448) as uint8."""
    return x.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()


def _pad_keys(vt: torch.Tensor, N: int) -> torch.Tensor:
    """[.., d, N] -> [.., d, Np] with Np = N rounded up to 16 (zero codes)."""
    Np = (N + 15) // 16 * 16
    out = torch.zeros(vt.shape[:-1] + (Np,), dtype=vt.dtype)
    out[..., :N] = vt
    return out.contiguous()


def fp8_inputs(B, Hq, Hkv, N, d, seed: int, kind: str = "normal"):
    """Seeded 8-bit (q8, k8, vt8, q_scale, k_scale, v_scale) on the CPU.

    kind "normal": i.i.d. N(0,1) values, each tensor scaled so its largest
    magnitude maps to 224 and rounded to E4M3 (the decoded codes times the
    scale are the inputs).  kind "exact": q and k rows with three entries of
    +-1 at seeded positions (scale 1), so every score q.k is an integer in
    [-3, 3]; v i.i.d. normal as above.
    vt8 is V transposed, [B, Hkv, d, Np], its padding keys zero codes.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 17)
    v = _randn((B, Hkv, N, d), seed + 2)
    v_scale = float(v.abs().max()) / 224.0
    vt8 = _pad_keys(_e4m3_codes((v / v_scale).transpose(-1, -2)), N)
    if kind == "normal":
        q = _randn((B, Hq, N, d), seed + 0)
        k = _randn((B, Hkv, N, d), seed + 1)
        q_scale = float(q.abs().max()) / 224.0
        k_scale = float(k.abs().max()) / 224.0
        return _e4m3_codes(q / q_scale), _e4m3_codes(k / k_scale), vt8, q_scale, k_scale, v_scale
    if kind == "exact":
        def sparse_pm1(shape):
            x = torch.zeros(shape)
            idx = torch.stack([torch.randperm(d, generator=g)[:3] for _ in range(x.numel() // d)])
            sign = torch.randint(0, 2, idx.shape, generator=g).float() * 2.0 - 1.0
            x.view(-1, d).scatter_(1, idx, sign)
            return x
        q = sparse_pm1((B, Hq, N, d))
        k = sparse_pm1((B, Hkv, N, d))
        return _e4m3_codes(q), _e4m3_codes(k), vt8, 1.0, 1.0, v_scale
    raise ValueError(f"unknown kind {kind!r}")
