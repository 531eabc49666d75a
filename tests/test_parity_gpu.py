"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Run on an MI355X:  python -u -m pytest tests -m gpu -x -v
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import LSE_TOL, compare, half_ulp, round_to

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from exact_io_aware_73_amd import attn as a   # fails loudly if libattn.so is missing
    return a


def _say(*msg):
    print(*msg, file=sys.stderr, flush=True)


def _dt(dtype):
    return "bf16" if dtype == torch.bfloat16 else "f32"


def _run(attn, q, k, v, scale):
    o, lse = attn.fwd(q.cuda(), k.cuda(), v.cuda(), scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _check_full(attn, q, k, v, scale, dtype, label):
    _say(f"[parity] {label} q={tuple(q.shape)} k={tuple(k.shape)} {dtype} scale={scale}")
    o, lse = _run(attn, q, k, v, scale)
    O_ref, lse_ref = oracle.attention_ref(workloads.to_f64(q), workloads.to_f64(k),
                                          workloads.to_f64(v), scale)
    r = compare(workloads.to_f64(o), lse.numpy(), O_ref, lse_ref, _dt(dtype))
    assert r["ok"], (label, r)
    return r


# ---------------------------------------------------------------------------
# small and ragged shapes: every tile edge, the tail, GQA groupings
SMALL_N = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 200, 1000]
HEADS = [(1, 1, 1), (1, 4, 1), (2, 8, 2)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", SMALL_N)
@pytest.mark.parametrize("B,Hq,Hkv", HEADS)
def test_fused_bf16_small(attn, B, Hq, Hkv, N, d):
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, torch.bfloat16, seed=7 * N + d + Hq)
    _check_full(attn, q, k, v, 1.0 / math.sqrt(d), torch.bfloat16, "fused bf16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 3, 31, 32, 33, 64, 65, 200, 1000])
@pytest.mark.parametrize("B,Hq,Hkv", HEADS)
def test_fused_f32_small(attn, B, Hq, Hkv, N, d):
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, torch.float32, seed=11 * N + d + Hq)
    _check_full(attn, q, k, v, 1.0 / math.sqrt(d), torch.float32, "fused f32")


# The query heads of a K/V group are packed into shared query tiles: tiles
# that cross head boundaries, groups of more rows than a tile, one row per head.
PACKED = [(1, 16, 1, 1), (1, 16, 1, 33), (2, 12, 3, 100), (1, 32, 4, 77), (1, 8, 8, 45), (1, 4, 2, 300)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,Hq,Hkv,N", PACKED)
def test_fused_bf16_gqa_packed(attn, B, Hq, Hkv, N, d):
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, torch.bfloat16, seed=19 * N + d + Hq)
    _check_full(attn, q, k, v, 1.0 / math.sqrt(d), torch.bfloat16, "packed GQA bf16")


@pytest.mark.parametrize("B,Hq,Hkv,N", PACKED[1:4])
def test_split_gqa_packed(attn, B, Hq, Hkv, N):
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, 128, torch.bfloat16, seed=23 * N + Hq)
    scale = 1.0 / math.sqrt(128)
    _say(f"[parity] split packed q={tuple(q.shape)} k={tuple(k.shape)}")
    o, lse = attn.fwd_split(q.cuda(), k.cuda(), v.cuda(), 3, scale)
    torch.cuda.synchronize()
    O_ref, lse_ref = oracle.attention_ref(workloads.to_f64(q), workloads.to_f64(k),
                                          workloads.to_f64(v), scale)
    r = compare(workloads.to_f64(o.cpu()), lse.cpu().numpy(), O_ref, lse_ref, "bf16")
    assert r["ok"], r


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [512, 500])
def test_many_workgroups(attn, N, d):
    """More workgroups than the GPU holds at once (d = 128: 320 workgroups of
    256 rows), with whole (512) and partial (500) last key tiles, GQA g = 4."""
    q, k, v = workloads.random_inputs(1, 160, 40, N, d, torch.bfloat16, seed=13 * N + d)
    _check_full(attn, q, k, v, 1.0 / math.sqrt(d), torch.bfloat16, "many workgroups")


# ---------------------------------------------------------------------------
# split-KV path: key ranges per workgroup, partial (O, lse) merged
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,n_split", [(1, 1), (1, 4), (31, 2), (32, 2), (33, 2), (100, 3),
                                        (257, 4), (1000, 7), (1000, 64)])
@pytest.mark.parametrize("B,Hq,Hkv", [(1, 1, 1), (2, 8, 2)])
def test_split_small(attn, B, Hq, Hkv, N, n_split, d):
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, torch.bfloat16, seed=17 * N + d + n_split)
    scale = 1.0 / math.sqrt(d)
    _say(f"[parity] split n_split={n_split} q={tuple(q.shape)} k={tuple(k.shape)}")
    o, lse = attn.fwd_split(q.cuda(), k.cuda(), v.cuda(), n_split, scale)
    torch.cuda.synchronize()
    O_ref, lse_ref = oracle.attention_ref(workloads.to_f64(q), workloads.to_f64(k),
                                          workloads.to_f64(v), scale)
    r = compare(workloads.to_f64(o.cpu()), lse.cpu().numpy(), O_ref, lse_ref, "bf16")
    assert r["ok"], r


@pytest.mark.parametrize("scale", [-0.09, 0.0, 3.0])
def test_split_scales(attn, scale):
    q, k, v = workloads.random_inputs(1, 4, 2, 300, 128, torch.bfloat16, seed=98)
    o, lse = attn.fwd_split(q.cuda(), k.cuda(), v.cuda(), 3, scale)
    torch.cuda.synchronize()
    O_ref, lse_ref = oracle.attention_ref(workloads.to_f64(q), workloads.to_f64(k),
                                          workloads.to_f64(v), scale)
    r = compare(workloads.to_f64(o.cpu()), lse.cpu().numpy(), O_ref, lse_ref, "bf16")
    assert r["ok"], r


def test_split_single_long_head(attn):
    """One head of 32768 rows (128 workgroups unsplit): four key ranges,
    sampled rows against the oracle, every row against the unsplit path."""
    q, k, v = workloads.random_inputs(1, 1, 1, 32768, 128, torch.bfloat16, seed=21)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    _say("[parity] split single head N=32768 n_split=4")
    o1, l1 = attn.fwd_split(qd, kd, vd, 4)
    o2, l2 = attn.fwd_split(qd, kd, vd, 4)
    o0, l0 = attn.fwd(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "not deterministic"
    # both paths approximate the same exact result within the bf16 bound
    assert (o1.float() - o0.float()).abs().max().item() <= 2e-2
    assert (l1 - l0).abs().max().item() <= 2e-3
    r = check_sampled(q, k, v, o1.cpu(), l1.cpu(), 1 / math.sqrt(128), "bf16", seed=5)
    _say(f"[parity] split single head: {r}")


def test_python_split_rejects(attn):
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        attn.fwd_split(q, q, q, 0)
    with pytest.raises(ValueError):
        attn.fwd_split(q, q, q, attn.ATTN_MAX_SPLIT + 1)
    o = torch.empty_like(q)
    lse = torch.empty(1, 2, 8, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")   # far too small
    with pytest.raises(ValueError):
        attn.attn_fwd_split(q, q, q, o, lse, ws, 2, 0.125)


def test_single_head_fp32_workload(attn):
    w = workloads.WORKLOADS["single_head_n256_d64_f32"]
    q, k, v = workloads.make_inputs(w)
    r = _check_full(attn, q, k, v, 1.0 / math.sqrt(w.d), torch.float32, w.name)
    assert r["max_abs_O"] <= 1e-4 and r["max_abs_lse"] <= 1e-3


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5, 3.0])
def test_fused_scales(attn, dtype, scale):
    """Zero, negative and large scales (any finite scale is allowed)."""
    q, k, v = workloads.random_inputs(1, 4, 2, 300, 128, dtype, seed=99)
    _check_full(attn, q, k, v, scale, dtype, f"scale {scale}")


def test_fused_wide_inputs(attn):
    """Scores spread over hundreds: the running max moves often and far."""
    q, k, _ = workloads.random_inputs(1, 2, 1, 700, 64, torch.bfloat16, seed=5, std=6.0)
    _, _, v = workloads.random_inputs(1, 2, 1, 700, 64, torch.bfloat16, seed=6)
    _check_full(attn, q, k, v, 1.0 / 8, torch.bfloat16, "wide scores")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("pattern", ["ramp", "steps", "falling"])
def test_fused_moving_max(attn, pattern, d):
    """Row maxima that keep growing along the keys (a ramp of key norms, or
    each 64-key tile's keys doubled against the previous tile's), so the
    kernels' bound on the weights keeps failing mid-row and the running max
    is moved and the accumulators rescaled on later tiles; and the reverse,
    maxima that only fall, where the first tile's max bounds the rest."""
    N = 1000
    q, k, v = workloads.random_inputs(1, 2, 1, N, d, torch.bfloat16, seed=41)
    j = torch.arange(N, dtype=torch.float32)
    if pattern == "ramp":
        f = 1.0 + j / 64.0
    elif pattern == "steps":
        f = 2.0 ** torch.clamp(j // 64, max=6)
    else:
        f = 2.0 ** -torch.clamp(j // 64, max=6) * 8.0
    k = (k.float() * f[None, None, :, None]).to(torch.bfloat16)
    _check_full(attn, q, k, v, 1.0 / math.sqrt(d), torch.bfloat16, f"moving max {pattern}")


# ---------------------------------------------------------------------------
# invariants through the GPU
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gpu_scale_zero_gives_mean(attn, dtype):
    q, k, v = workloads.random_inputs(2, 4, 2, 333, 64, dtype, seed=3)
    o, lse = _run(attn, q, k, v, 0.0)
    mean = workloads.to_f64(v).mean(axis=2, keepdims=True).repeat(2, axis=1)
    tol = 1e-2 if dtype == torch.bfloat16 else 1e-4
    assert np.max(np.abs(workloads.to_f64(o) - mean)) <= tol + half_ulp(mean, _dt(dtype)).max()
    assert np.max(np.abs(lse.numpy() - math.log(333))) <= LSE_TOL


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gpu_single_key(attn, dtype):
    """N = 1: O = V_0 exactly (one weight of exactly 1), lse = scale q.k_0."""
    q, k, v = workloads.random_inputs(3, 4, 4, 1, 128, dtype, seed=4)
    o, lse = _run(attn, q, k, v, 0.3)
    assert torch.equal(o, v)
    ref = 0.3 * np.einsum("bhnd,bhnd->bhn", workloads.to_f64(q), workloads.to_f64(k))
    assert np.max(np.abs(lse.numpy() - ref)) <= LSE_TOL


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gpu_constant_v(attn, dtype):
    q, k, _ = workloads.random_inputs(1, 2, 1, 517, 128, dtype, seed=6)
    row = torch.randn(1, 1, 1, 128, generator=torch.Generator().manual_seed(1)).to(dtype)
    v = row.expand(1, 1, 517, 128).contiguous()
    o, _ = _run(attn, q, k, v, 1 / math.sqrt(128))
    ref = workloads.to_f64(row).repeat(2, axis=1)
    tol = 1e-2 if dtype == torch.bfloat16 else 1e-4
    assert np.max(np.abs(workloads.to_f64(o) - ref)) <= tol


def test_gpu_one_hot(attn):
    """A key far ahead of all others selects its V row."""
    N, d = 256, 64
    q = torch.zeros(1, 1, N, d)
    k = torch.rand(1, 1, N, d, generator=torch.Generator().manual_seed(2)) - 0.5
    for c in range(d):
        k[0, 0, 3 * c] = 0.0
        k[0, 0, 3 * c, c] = 8.0
    for i in range(N):
        q[0, 0, i, i % d] = 8.0
    v = torch.randn(1, 1, N, d, generator=torch.Generator().manual_seed(3))
    q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    o, _ = _run(attn, q, k, v, 1.0)   # winner 64, others <= 4
    for i in range(N):
        assert torch.equal(o[0, 0, i], v[0, 0, 3 * (i % d)])


def test_gpu_gqa_equals_repeated_heads(attn):
    """GQA equals MHA on repeated K/V heads, bit for bit."""
    q, k, v = workloads.random_inputs(2, 8, 2, 777, 128, torch.bfloat16, seed=8)
    o1, l1 = _run(attn, q, k, v, 0.1)
    o2, l2 = _run(attn, q, k.repeat_interleave(4, dim=1).contiguous(),
                  v.repeat_interleave(4, dim=1).contiguous(), 0.1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gpu_shift_keys(attn):
    """K' = K + u: compare against the oracle on the same (re-rounded) K'."""
    q, k, v = workloads.random_inputs(1, 2, 2, 400, 128, torch.bfloat16, seed=10)
    u = torch.randn(128, generator=torch.Generator().manual_seed(11)) * 2
    k2 = (k.float() + u).bfloat16().contiguous()
    _check_full(attn, q, k2, v, 1 / math.sqrt(128), torch.bfloat16, "shifted K")


def test_gpu_deterministic_and_stream(attn):
    q, k, v = workloads.random_inputs(2, 8, 2, 1500, 128, torch.bfloat16, seed=12)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = attn.fwd(q, k, v)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = attn.fwd(q, k, v, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_python_rejects_bad_arguments(attn):
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        attn.fwd(q, k[:, :, :4].contiguous(), k)
    with pytest.raises(ValueError):
        attn.fwd(q, k, k, scale=float("nan"))
    with pytest.raises(ValueError):
        attn.fwd(torch.zeros(1, 2, 8, 96, dtype=torch.bfloat16, device="cuda"),
                 torch.zeros(1, 1, 8, 96, dtype=torch.bfloat16, device="cuda"),
                 torch.zeros(1, 1, 8, 96, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        attn.fwd(q.half(), k.half(), k.half())


# ---------------------------------------------------------------------------
# materialising path: O, lse, and the S and P it writes
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
# N covers the three row-softmax kernels of the comparison path: N % 4 != 0
# (one score per thread), N % 4 == 0 up to 4096 (one wave per row, from
# registers) and beyond (two passes of 16-byte loads)
@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(1, 1, 1, 1, 64), (1, 2, 1, 37, 64), (2, 4, 2, 129, 128),
                                           (1, 2, 2, 256, 64), (1, 4, 1, 300, 128), (1, 1, 1, 1000, 64),
                                           (1, 1, 1, 4100, 64)])
def test_materialized_small(attn, dtype, B, Hq, Hkv, N, d):
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, dtype, seed=13 * N + d)
    scale = 1 / math.sqrt(d)
    _say(f"[parity] materialized {dtype} {(B, Hq, Hkv, N, d)}")
    o, lse, s, p = attn.fwd_materialized(q.cuda(), k.cuda(), v.cuda(), scale)
    torch.cuda.synchronize()
    O_ref, lse_ref, S_ref, P_ref = oracle.attention_ref_sp(
        workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v), scale)
    r = compare(workloads.to_f64(o), lse.cpu().numpy(), O_ref, lse_ref, _dt(dtype))
    assert r["ok"], r
    s64 = s.cpu().double().numpy()
    p64 = workloads.to_f64(p)
    # S: fp32 accumulation of exact products; P: the I/O format's rounding
    assert np.max(np.abs(s64 - S_ref)) <= 1e-4
    assert np.max(np.abs(p64 - P_ref) - 2 * half_ulp(P_ref, _dt(dtype))) <= 1e-5


# ---------------------------------------------------------------------------
# the named workloads at full size, in the launch configuration bench.py
# times: sampled rows against the oracle, properties on every row, and
# bitwise determinism
FULL = ["gpt2_medium_b64_h16_n1024_d64", "long_b4_h32_n4096_d128", "gqa_b2_hq32_hkv8_n8192_d128",
        "gqa_b2_hq32_hkv8_n8192_d128_kscaled", "long_context_b1_h8_n32768_d128"]


def sample_rows(N, rng, n_rand=32):
    rows = set(range(min(16, N))) | set(range(max(0, N - 16), N))
    rows |= set(rng.choice(N, size=min(n_rand, N), replace=False).tolist())
    return sorted(rows)


def check_sampled(q, k, v, o, lse, scale, dtype, seed=0):
    """Oracle on sampled rows of three heads (first, last, one random)."""
    B, Hq, N, d = q.shape
    rng = np.random.default_rng(seed)
    heads = {(0, 0), (B - 1, Hq - 1), (int(rng.integers(B)), int(rng.integers(Hq)))}
    worst = None
    for (b, h) in sorted(heads):
        kv = oracle.kv_head(h, Hq, k.shape[1])
        rows = sample_rows(N, rng)
        O_ref, l_ref = oracle.attention_head(workloads.to_f64(q[b, h]), workloads.to_f64(k[b, kv]),
                                             workloads.to_f64(v[b, kv]), scale, rows=rows)
        r = compare(workloads.to_f64(o[b, h, rows]), lse[b, h, rows].numpy(), O_ref, l_ref, dtype)
        assert r["ok"], ((b, h), r)
        if worst is None or r["max_abs_O"] > worst["max_abs_O"]:
            worst = r
    return worst


def check_every_head(q, k, v, o, lse, scale, dtype, seed=0, n_rows=4):
    """Oracle on a few random rows of EVERY head."""
    B, Hq, N, d = q.shape
    rng = np.random.default_rng(seed + 1)
    for b in range(B):
        for kv in range(k.shape[1]):
            kk, vv = workloads.to_f64(k[b, kv]), workloads.to_f64(v[b, kv])
            g = Hq // k.shape[1]
            for h in range(kv * g, (kv + 1) * g):
                rows = sorted(rng.choice(N, size=min(n_rows, N), replace=False).tolist())
                O_ref, l_ref = oracle.attention_head(workloads.to_f64(q[b, h, rows]), kk, vv, scale)
                r = compare(workloads.to_f64(o[b, h, rows]), lse[b, h, rows].numpy(), O_ref, l_ref,
                            dtype)
                assert r["ok"], ((b, h), rows, r)


def _rows64_plan(attn, B, Hq, Hkv, N, d):
    kern = attn.attn_fwd_plan(B, Hq, Hkv, N, d)
    assert kern == attn.ATTN_KERNEL_ROWS64, (B, Hq, Hkv, N, d, kern)


def test_kernel_plan_by_shape(attn):
    """Which kernel each bf16 shape runs, asked of the library: rows64 where
    head dim 128, N >= 1024 and the 256-row grid has a workgroup per compute
    unit."""
    n_cu, n_xcd, l2 = attn.attn_device_info()
    _say(f"[parity] device: {n_cu} compute units, {n_xcd} XCDs, L2 {l2} bytes")
    assert n_cu >= 1 and n_xcd >= 1
    R32, R64 = attn.ATTN_KERNEL_ROWS32, attn.ATTN_KERNEL_ROWS64
    want = {"gpt2_medium_b64_h16_n1024_d64": R32, "gqa_short_b64_hq32_hkv4_n200_d128": R32}
    if n_cu <= 256:
        want.update({"gqa_b2_hq32_hkv8_n8192_d128": R64, "long_context_b1_h8_n32768_d128": R64,
                     "long_b4_h32_n4096_d128": R64})
    if n_cu > 128:
        want["one_head_b1_h1_n32768_d128"] = R32     # 128 workgroups of 256 rows
    for name, kern in want.items():
        w = workloads.WORKLOADS[name]
        assert attn.attn_fwd_plan(w.B, w.Hq, w.Hkv, w.N, w.d) == kern, name
    # the rule's edges: N, head dim, and the grid against the compute units
    rows_for = lambda g_rows: -(-g_rows // 256)        # 256-row workgroups of one group
    hkv = -(-n_cu // rows_for(4 * 8192))                 # just enough groups to fill the CUs
    assert attn.attn_fwd_plan(1, 4 * hkv, hkv, 8192, 128) == R64
    assert attn.attn_fwd_plan(1, 4 * hkv, hkv, 8192, 64) == R32
    if hkv > 1:
        assert attn.attn_fwd_plan(1, 4 * (hkv - 1), hkv - 1, 8192, 128) == R32
    h = -(-n_cu // rows_for(1024))                        # heads of 1024 rows filling the CUs
    assert attn.attn_fwd_plan(1, h, h, 1024, 128) == R64
    assert attn.attn_fwd_plan(1, h, h, 1023, 128) == R32
    assert attn.attn_fwd_plan(1, 2 * h, 2 * h, 1023, 128) == R32


@pytest.mark.parametrize("scale", [1 / math.sqrt(128), -0.05, 0.0])
def test_rows64_reversed_rounds(attn, scale):
    """N = 8192, head dim 128, a GQA group per K/V head: the keys fit one XCD's
    L2, so every other round of workgroups streams them in reverse order and
    stores O as whole rows through LDS.  1024 workgroups (four rounds), every
    head checked on sampled rows; bitwise deterministic."""
    B, Hq, Hkv, N, d = 1, 32, 8, 8192, 128
    _rows64_plan(attn, B, Hq, Hkv, N, d)
    _say(f"[parity] rows64 reversed rounds {B},{Hq},{Hkv},{N},{d} scale={scale}")
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, torch.bfloat16, seed=8192 + int(100 * scale))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = attn.fwd(qd, kd, vd, scale)
    o2, l2 = attn.fwd(qd, kd, vd, scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2), "not deterministic"
    o, lse = o.cpu(), lse.cpu()
    check_sampled(q, k, v, o, lse, scale, "bf16", seed=9)
    check_every_head(q, k, v, o, lse, scale, "bf16", seed=9, n_rows=16)


@pytest.mark.parametrize("scale", [1 / math.sqrt(128), -0.05])
def test_rows64_long_ragged(attn, scale):
    """Head dim 128 with N >= 1024 and a grid of at least one workgroup per CU
    runs the rows64 kernel (shorter keys or smaller grids run rows32): a
    ragged last key tile and a GQA group, sampled rows against the oracle."""
    B, Hq, Hkv, N, d = 1, 16, 4, 8197, 128
    _rows64_plan(attn, B, Hq, Hkv, N, d)
    _say(f"[parity] rows64 long ragged {B},{Hq},{Hkv},{N},{d} scale={scale}")
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, torch.bfloat16, seed=8197)
    o, lse = attn.fwd(q.cuda(), k.cuda(), v.cuda(), scale)
    torch.cuda.synchronize()
    check_sampled(q, k, v, o.cpu(), lse.cpu(), scale, "bf16", seed=5)


@pytest.mark.parametrize("N", [1024, 1500])
def test_rows64_short_keys(attn, N):
    """The shortest keys rows64 takes (N >= 1024, a full grid of GQA groups):
    whole and ragged last tiles, every head checked on sampled rows."""
    n_cu = attn.attn_device_info()[0]
    hkv = max(4, -(-n_cu // (-(-4 * N // 256))))
    B, Hq, Hkv, d = 1, 4 * hkv, hkv, 128
    _rows64_plan(attn, B, Hq, Hkv, N, d)
    _say(f"[parity] rows64 short keys {B},{Hq},{Hkv},{N},{d}")
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, torch.bfloat16, seed=N + 3)
    o, lse = attn.fwd(q.cuda(), k.cuda(), v.cuda(), 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    check_sampled(q, k, v, o, lse, 1.0 / math.sqrt(d), "bf16", seed=3)
    check_every_head(q, k, v, o, lse, 1.0 / math.sqrt(d), "bf16", seed=3, n_rows=8)


@pytest.mark.parametrize("N", [8192, 8200])
@pytest.mark.parametrize("pattern", ["ramp", "steps", "falling"])
def test_rows64_moving_max(attn, pattern, N):
    """The rows64 kernel's rescale path: key norms that ramp up or double
    every 1024 keys along a long row (the running max moves by more than the
    kernel's threshold on later tiles and the accumulators are rescaled), and
    the reverse, on a shape that runs rows64, every head checked on sampled
    rows.  N = 8192: a K/V head fits one XCD's L2, so alternate rounds of
    workgroups stream the keys in reverse order (both orders in one launch);
    N = 8200 has a partial last tile and keeps the forward order."""
    B, Hq, Hkv, d = 1, 16, 4, 128
    _rows64_plan(attn, B, Hq, Hkv, N, d)
    _say(f"[parity] rows64 moving max {pattern} {B},{Hq},{Hkv},{N},{d}")
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, torch.bfloat16, seed=N)
    j = torch.arange(N, dtype=torch.float32)
    if pattern == "ramp":
        f = 1.0 + j / 512.0
    elif pattern == "steps":
        f = 2.0 ** torch.clamp(j // 1024, max=6)
    else:
        f = 2.0 ** -torch.clamp(j // 1024, max=6) * 8.0
    k = (k.float() * f[None, None, :, None]).to(torch.bfloat16).contiguous()
    scale = 1 / math.sqrt(d)
    o, lse = attn.fwd(q.cuda(), k.cuda(), v.cuda(), scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    check_sampled(q, k, v, o, lse, scale, "bf16", seed=6)
    check_every_head(q, k, v, o, lse, scale, "bf16", seed=6, n_rows=8)


@pytest.mark.parametrize("name", FULL)
def test_full_workload(attn, name):
    w = workloads.WORKLOADS[name]
    _say(f"[parity] full workload {name}")
    q, k, v = workloads.make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    scale = 1 / math.sqrt(w.d)
    o1, l1 = attn.fwd(qd, kd, vd, scale)
    o2, l2 = attn.fwd(qd, kd, vd, scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "not deterministic"
    # every row: finite, a convex combination of V rows, lse >= the row max
    assert torch.isfinite(o1).all() and torch.isfinite(l1).all()
    vmax = vd.float().abs().amax(dim=(2, 3))                         # [B, Hkv]
    vmax = vmax.repeat_interleave(w.Hq // w.Hkv, dim=1)[:, :, None, None]
    assert (o1.float().abs() <= vmax * (1 + 2 ** -6) + 1e-6).all()
    o, lse = o1.cpu(), l1.cpu()
    del o1, o2, l1, l2
    r = check_sampled(q, k, v, o, lse, scale, w.dtype, seed=w.seed)
    check_every_head(q, k, v, o, lse, scale, w.dtype, seed=w.seed)
    _say(f"[parity] {name}: {r}")


def test_materialized_long_workload(attn):
    """The long-sequence workload through the materialising path (S is 8.6 GB)."""
    w = workloads.WORKLOADS["long_b4_h32_n4096_d128"]
    _say("[parity] materialized full long workload")
    q, k, v = workloads.make_inputs(w)
    scale = 1 / math.sqrt(w.d)
    o, lse, s, p = attn.fwd_materialized(q.cuda(), k.cuda(), v.cuda(), scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = sample_rows(w.N, rng, 8)
    for (b, h) in [(0, 0), (w.B - 1, w.Hq - 1)]:
        qh, kh, vh = (workloads.to_f64(t[b, h]) for t in (q, k, v))
        S_ref = oracle.head_scores(qh[rows], kh, scale)
        P_ref, l_ref = oracle.softmax_rows(S_ref)
        O_ref = P_ref @ vh
        assert np.max(np.abs(s[b, h, rows].cpu().double().numpy() - S_ref)) <= 1e-4
        p64 = workloads.to_f64(p[b, h, rows])
        assert np.max(np.abs(p64 - P_ref) - 2 * half_ulp(P_ref, "bf16")) <= 1e-5
        r = compare(workloads.to_f64(o[b, h, rows]), lse[b, h, rows].cpu().numpy(), O_ref, l_ref, "bf16")
        assert r["ok"], r
    del s, p


# ---------------------------------------------------------------------------
# seeded random shapes across both kernels and both key orders: head counts,
# GQA ratios, ragged N on either side of the rows64 threshold, both signs of
# scale; every head checked on a few rows, three heads on more
def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.integers(1, 9))
        B = int(rng.integers(1, 4))
        N = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(900, 1200)),
                            int(rng.integers(1500, 6000)), 4096, 8192]))
        scale = float(rng.choice([1.0 / math.sqrt(d), -0.07, 0.3]))
        shapes.append((B, g * hkv, hkv, N, d, scale, 1000 + i))
    return shapes


@pytest.mark.parametrize("B,Hq,Hkv,N,d,scale,seed", _random_shapes(16, 20261203))
def test_random_shapes(attn, B, Hq, Hkv, N, d, scale, seed):
    _say(f"[parity] random shape {B},{Hq},{Hkv},{N},{d} scale={scale:.3f} "
         f"plan={attn.attn_fwd_plan(B, Hq, Hkv, N, d)}")
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, torch.bfloat16, seed=seed)
    o, lse = attn.fwd(q.cuda(), k.cuda(), v.cuda(), scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    check_sampled(q, k, v, o, lse, scale, "bf16", seed=seed)
    check_every_head(q, k, v, o, lse, scale, "bf16", seed=seed, n_rows=2)


def _random_rows64_shapes(n, seed):
    """Head dim 128, N >= 1024 and enough K/V groups to fill 256 compute units
    with 256-row workgroups: the rows64 kernel, ragged and whole last tiles,
    groups spanning one or several rounds (the reversed key order)."""
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        g = int(rng.choice([1, 2, 4, 8]))
        N = int(rng.choice([int(rng.integers(1024, 9000)), 32 * int(rng.integers(32, 300))]))
        per_group = -(-g * N // 256)
        groups = -(-256 // per_group) + int(rng.integers(0, 3))
        B = 1 + int(rng.integers(0, 2))
        hkv = -(-groups // B)
        scale = float(rng.choice([1.0 / math.sqrt(128), -0.07, 0.3]))
        shapes.append((B, g * hkv, hkv, N, 128, scale, 2000 + i))
    return shapes


@pytest.mark.parametrize("B,Hq,Hkv,N,d,scale,seed", _random_rows64_shapes(8, 1203))
def test_random_rows64_shapes(attn, B, Hq, Hkv, N, d, scale, seed):
    n_cu = attn.attn_device_info()[0]
    if n_cu <= 256:
        _rows64_plan(attn, B, Hq, Hkv, N, d)
    test_random_shapes(attn, B, Hq, Hkv, N, d, scale, seed)
