"""Benchmark: exact attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

One step = one launch of the fused forward (attn_fwd) over the workload's
whole batch, inputs resident in HBM.  Prints ONE JSON line with throughput
(TFLOP/s, 4*B*Hq*N^2*d FLOPs), the roofline position of the kernel (timed
with HIP events on its own stream), the materialising path's time beside
it, the HBM traffic taken from committed rocprofv3 counter summaries (when
they match the current kernel source), and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads  # noqa: E402
from exact_io_aware_73_amd import accounting as acc  # noqa: E402

METRIC = "attention fwd TFLOP/s and % of bf16 MFMA peak; HBM bytes vs Q/K/V/O min"
# the sources each workload's fused kernel is built from, by I/O dtype and head dim
_COMMON_SOURCES = ["exact_io_aware_73_amd/csrc/device_common.hpp"]


def _hash_sources(rels) -> str:
    """Hash of the given sources, the shared header and the compile flags
    that apply to them (the global flags and each file's own), so an edit to
    another file's flags leaves the hash alone."""
    from exact_io_aware_73_amd import build as B
    h = hashlib.sha256()
    for rel in list(rels) + _COMMON_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    flags = [" ".join(B.CFLAGS)] + [f"{os.path.basename(r)}: {' '.join(B.FILE_FLAGS.get(os.path.basename(r), []))}"
                                    for r in rels]
    h.update("\n".join(flags).encode())
    return h.hexdigest()[:16]
KERNEL_SOURCES = {
    ("bf16", 64): ["exact_io_aware_73_amd/csrc/attn_fwd_bf16_rows32.hip"],
    # head dim 128 runs rows64 or rows32 by shape (the rule is in kernels.hpp)
    ("bf16", 128): ["exact_io_aware_73_amd/csrc/attn_fwd_bf16_rows64.hip",
                    "exact_io_aware_73_amd/csrc/rows64_pipeline.hpp",
                    "exact_io_aware_73_amd/csrc/attn_fwd_bf16_rows32.hip",
                    "exact_io_aware_73_amd/csrc/kernels.hpp"],
    ("f32", 64): ["exact_io_aware_73_amd/csrc/attn_fwd_f32.hip"],
    ("f32", 128): ["exact_io_aware_73_amd/csrc/attn_fwd_f32.hip"],
}


def kernel_source_hash(workload: str) -> str:
    """Hash of the sources of the kernel that runs `workload` (a counter
    summary taken on other sources no longer describes that kernel)."""
    w = workloads.ALL[workload]
    return _hash_sources(KERNEL_SOURCES[(w.dtype, w.d)])


# the sources of the three kernels of the materialising path
MATERIALIZED_SOURCES = ["exact_io_aware_73_amd/csrc/attn_materialized.hip",
                        "exact_io_aware_73_amd/csrc/bf16_tiles.hpp"]


def materialized_source_hash() -> str:
    return _hash_sources(MATERIALIZED_SOURCES)


def _counters(path: str, sha: str):
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != sha:
        return None
    return rec


def traffic_from_profiles(workload: str, per_launch_flops: int = 0, profiles_dir: str | None = None):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, or None when absent or taken on other kernel source."""
    rec = _counters(os.path.join(profiles_dir or os.path.join(ROOT, "profiles"),
                                 f"attn_fwd_{workload}_counters.json"), kernel_source_hash(workload))
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def materialized_traffic_from_profiles(workload: str, profiles_dir: str | None = None):
    """(read, write) bytes per call of the materialising path (its three
    kernels summed) from the committed counter summary, or None."""
    rec = _counters(os.path.join(profiles_dir or os.path.join(ROOT, "profiles"),
                                 f"attn_fwd_materialized_{workload}_counters.json"),
                    materialized_source_hash())
    if rec is None:
        return None
    return rec["hbm_read_bytes_per_launch"], rec["hbm_write_bytes_per_launch"]


# the sources of the backward's kernels (row dot, dK/dV, dQ)
BACKWARD_SOURCES = ["exact_io_aware_73_amd/csrc/attn_bwd.hip", "exact_io_aware_73_amd/csrc/kernels.hpp"]


def backward_source_hash() -> str:
    return _hash_sources(BACKWARD_SOURCES)


def backward_traffic_from_profiles(workload: str, profiles_dir: str | None = None):
    """(read, write) bytes per call of the backward (its kernels summed) from
    the committed counter summary, or None."""
    rec = _counters(os.path.join(profiles_dir or os.path.join(ROOT, "profiles"),
                                 f"attn_bwd_{workload}_counters.json"), backward_source_hash())
    if rec is None:
        return None
    return rec["hbm_read_bytes_per_launch"], rec["hbm_write_bytes_per_launch"]


def warm_up(fn, warmup: int, min_ms: float):
    """`warmup` launches, then more until at least `min_ms` of wall time has
    been spent launching: the GPU runs its first tens of milliseconds of work
    at a lower clock, so a count of launches alone does not warm it at short
    workloads.  Returns (launches run, wall ms)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn()
        n += 1
        if n >= warmup and n % 4 == 0:
            torch.cuda.synchronize()   # let the wall clock see the work, not the enqueue
    torch.cuda.synchronize()
    return n, (time.perf_counter() - t0) * 1e3


def time_launches(fn, stream, steps: int, warmup: int, min_warm_ms: float = 0.0):
    """Wall time of `steps` launches (synchronised on both sides) and the
    mean per-launch duration from HIP events recorded on `stream`."""
    warm_up(fn, warmup, min_warm_ms)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall / steps * 1e3, float(np.mean(ev)), float(np.min(ev)), float(np.median(ev))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, q, k, v, scale, budget_s: float = 12.0, threads: int = 16):
    """The fp64 oracle, as it stands, on the host cores, over a bounded sample
    of the same inputs: units of whole query rows of one head (all of a
    head's rows when a head is small, blocks of rows of ~1 GFLOP when it is
    long), handed in order to a pool of `threads` workers (single-threaded
    BLAS each) until the time budget is spent, passing over the workload
    again when it finishes sooner.  The rate counts the units completed."""
    import oracle
    from threadpoolctl import threadpool_limits
    from concurrent.futures import FIRST_COMPLETED, ThreadPoolExecutor, wait
    B, Hq, Hkv, N, d = w.B, w.Hq, w.Hkv, w.N, w.d
    rows = max(1, min(N, (1 << 30) // (4 * N * d)))
    units = [(b, h, r0, min(N, r0 + rows)) for b in range(B) for h in range(Hq)
             for r0 in range(0, N, rows)]
    import functools
    import threading
    lock = threading.Lock()

    @functools.lru_cache(maxsize=2 * threads)
    def kv64(b, kv):   # a K/V head as float64, shared by the units that read it
        return workloads.to_f64(k[b, kv]), workloads.to_f64(v[b, kv])

    def run(u):
        b, h, r0, r1 = u
        with lock:
            kk, vv = kv64(b, oracle.kv_head(h, Hq, Hkv))
        oracle.attention_head(workloads.to_f64(q[b, h, r0:r1]), kk, vv, scale)
        return r1 - r0

    done_rows = 0
    n_units = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(threads) as ex:
        pending = set()
        i = 0
        while True:
            while len(pending) < threads and time.perf_counter() - t0 < budget_s:
                pending.add(ex.submit(run, units[i % len(units)]))
                i += 1
            if not pending:
                break
            fin, pending = wait(pending, return_when=FIRST_COMPLETED)
            for fu in fin:
                done_rows += fu.result()
                n_units += 1
    t = time.perf_counter() - t0
    flops = 4 * done_rows * N * d
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"{n_units} units of up to {rows} query rows x all {N} keys "
                       f"({done_rows / (B * Hq * N):.3f} of the workload's rows) of {w.name}, "
                       f"fp64 NumPy, {threads} worker threads, {t:.1f} s"),
            "seconds": round(t, 3), "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


def mfma_ceiling(step_zero, stream, flops, steps: int):
    """Context for the roofline: what dense bf16 MFMA work reaches on this
    device with the same kind of data.  A library GEMM (8192^3, N(0,1)
    inputs) gives the practical ceiling under the chip's power limit; the
    fused kernel on all-zero inputs of the same shape shows how much of the
    gap to the nominal peak is data-dependent (power) rather than code."""
    g = torch.Generator(device="cuda").manual_seed(7)
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    with torch.cuda.stream(stream):
        gemm_ms, pw_gemm = sustained(lambda: torch.matmul(a, b, out=c), stream)
        zero_ms, pw_zero = sustained(step_zero, stream)
    gemm = 2.0 * n ** 3 / (gemm_ms * 1e-3) / 1e12
    del a, b, c
    return {"gemm": "torch.matmul bf16 8192x8192x8192, N(0,1) inputs", "gemm_tflops": round(gemm, 1),
            "gemm_frac_of_peak": round(gemm / acc.PEAK_BF16_TFLOPS, 4), "gemm_power_clock": pw_gemm,
            "attn_zero_inputs_tflops": round(flops / (zero_ms * 1e-3) / 1e12, 1),
            "attn_zero_inputs_power_clock": pw_zero}


def sustained(fn, stream, secs: float = 1.2):
    """`fn` launched back to back for `secs` seconds with power and clock
    sampled meanwhile (the device's metrics lag by tens of milliseconds, so
    the summary keeps the later samples); returns (mean ms per launch over
    the last half, the power / clock summary)."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    with PowerSampler() as pw:
        t0 = time.perf_counter()
        half = None
        n = 0
        while True:
            fn()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
                el = time.perf_counter() - t0
                if half is None and el >= secs / 2:
                    half = (n, torch.cuda.Event(enable_timing=True))
                    half[1].record(stream)
                if el >= secs:
                    break
        end = torch.cuda.Event(enable_timing=True)
        end.record(stream)
        torch.cuda.synchronize()
    ms = half[1].elapsed_time(end) / (n - half[0])
    return ms, pw.summary()


class PowerSampler:
    """Socket power and graphics clock of GPU 0 (amdsmi), sampled every few
    milliseconds while the `with` block runs; summary() gives their means
    over the later half of the samples (or None without amdsmi)."""

    def __init__(self, period_s: float = 0.005):
        self.period = period_s
        self.samples = []
        self._stop = None
        self._thread = None
        self._h = None

    def __enter__(self):
        import threading
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self._amdsmi = amdsmi
        except Exception:
            return self
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                try:
                    m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._h)
                    self.samples.append((float(m["current_socket_power"]), float(m["current_gfxclk"])))
                except Exception:
                    pass
                time.sleep(self.period)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        s = self.samples[len(self.samples) // 2:]
        if not s:
            return None
        return {"socket_power_w": round(sum(x for x, _ in s) / len(s), 1),
                "gfxclk_mhz": round(sum(y for _, y in s) / len(s), 1), "samples": len(s)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU needs tens of milliseconds of work to reach its running clock,
    # so the default warm-up is long enough for that at every workload
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=workloads.DEFAULT_BENCH, choices=sorted(workloads.ALL))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-materialized", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--cpu-threads", type=int, default=min(len(os.sched_getaffinity(0)), 16),
                    help="worker threads of the CPU oracle baseline")
    ap.add_argument("--min-warmup-ms", type=float, default=200.0,
                    help="keep launching warm-up steps until this much wall time has passed "
                         "(the clock settles over the first tens of milliseconds of work)")
    ap.add_argument("--split", type=int, default=0,
                    help="time the split-KV entry point (attn_fwd_split) with this many key "
                         "ranges instead of attn_fwd (bf16 only)")
    ap.add_argument("--backward", action="store_true",
                    help="also time attn_bwd (gradients of the same forward; bf16 only)")
    ap.add_argument("--fp8", action="store_true",
                    help="time the 8-bit entry point (attn_fwd_fp8) on the workload's shape: "
                         "E4M3 codes of seeded N(0,1) values with per-tensor scales")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the second of sustained launches that samples power and clock")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the library-GEMM / zero-input context measurement")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times): the "
                         "calibration kernel for the HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(each (batch, K/V-head) group is independent, so the design shards them "
              "across GPUs with no exchange, but that is not built).", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n}), flush=True)
        return

    from exact_io_aware_73_amd import attn

    w = workloads.ALL[args.workload]
    torch.cuda.set_device(0)
    q, k, v = workloads.make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    scale = 1.0 / math.sqrt(w.d)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    entry = attn.attn_fwd if w.dtype == "bf16" else attn.attn_fwd_f32
    if args.split:
        if w.dtype != "bf16":
            sys.exit("--split takes a bf16 workload")
        ws = torch.empty(attn.attn_fwd_split_workspace_bytes(w.B, w.Hq, w.N, w.d, args.split),
                         dtype=torch.uint8, device="cuda")

        def entry(q_, k_, v_, o_, lse_, scale_, stream_):
            attn.attn_fwd_split(q_, k_, v_, o_, lse_, ws, args.split, scale_, stream_)

    fp8 = None
    if args.fp8:
        if w.dtype != "bf16" or args.split or args.backward:
            sys.exit("--fp8 takes a bf16 workload's shape and runs the 8-bit forward alone")
        fp8 = workloads.fp8_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed)
        q8d, k8d, vt8d = (t.cuda() for t in fp8[:3])
        q_s, k_s, v_s = fp8[3:]

        def entry(q_, k_, v_, o_, lse_, scale_, stream_):
            attn.attn_fwd_fp8(q8d, k8d, vt8d, o_, lse_, q_s, k_s, v_s, scale_, stream_)

    def step():
        entry(qd, kd, vd, o, lse, scale, stream)

    with torch.cuda.stream(stream):
        n_warm, warm_ms = warm_up(step, args.warmup, args.min_warmup_ms)
        ms_step, ev_mean, ev_min, ev_med = time_launches(step, stream, args.steps, 0)
        # the clock and power the kernel runs at, sampled over a further second
        # of back-to-back launches (the timed steps may be too short to sample)
        sus_ms, power = sustained(step, stream) if not args.no_power else (None, None)
    n_cu, n_xcd, l2_bytes = attn.attn_device_info()
    kernel = ("attn_fwd_f32_kernel" if w.dtype != "bf16" else
              "attn_fwd_fp8_kernel" if fp8 else
              "attn_fwd_bf16_rows64_split_kernel + attn_split_merge_kernel" if args.split else
              {attn.ATTN_KERNEL_ROWS32: "attn_fwd_bf16_rows32_kernel",
               attn.ATTN_KERNEL_ROWS64: "attn_fwd_bf16_rows64_kernel"}[
                   attn.attn_fwd_plan(w.B, w.Hq, w.Hkv, w.N, w.d)] + f"<{w.d}>")

    flops = acc.attn_fwd_flops(w.B, w.Hq, w.N, w.d)
    minb = acc.min_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, w.elem_bytes)
    value = flops / (ms_step * 1e-3) / 1e12
    peak = (acc.PEAK_FP8_TFLOPS if fp8 else
            acc.PEAK_BF16_TFLOPS if w.dtype == "bf16" else acc.PEAK_FP32_VECTOR_TFLOPS)
    achieved = flops / (ev_mean * 1e-3) / 1e12
    # the byte counters are taken on attn_fwd; the split and 8-bit paths have their own kernels
    traffic = None if (args.split or fp8) else traffic_from_profiles(w.name, flops)
    roofline = {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic, "kernel": kernel, "kernel_ms_mean": round(ev_mean, 4),
                "kernel_ms_min": round(ev_min, 4), "kernel_ms_median": round(ev_med, 4),
                "min_bytes": minb,
                "traffic_vs_min": (round(traffic / minb, 3) if traffic else None),
                # achieved HBM bandwidth: the counted bytes over the mean kernel time
                "hbm_gbps": (round(traffic / (ev_mean * 1e-3) / 1e9, 1) if traffic else None),
                "hbm_frac": (round(traffic / (ev_mean * 1e-3) / 1e9 / acc.PEAK_HBM_GBPS, 4)
                             if traffic else None),
                "device": {"compute_units": n_cu, "xcds": n_xcd, "l2_bytes": l2_bytes},
                # the clock the kernel runs at (the peak assumes 2.4 GHz)
                "power_clock": (dict(power or {}, sustained_tflops=round(flops / (sus_ms * 1e-3) / 1e12, 1))
                                if sus_ms else None)}
    if w.dtype == "bf16" and not fp8 and w.d == 128 and w.N >= 4096:
        # the stated goals at N >= 4096, d = 128: half the bf16 peak, and at
        # most 1.5x the Q/K/V/O bytes
        roofline["targets"] = {
            "frac_at_least": 0.5, "frac_met": achieved / peak >= 0.5,
            "traffic_vs_min_at_most": 1.5,
            "traffic_met": (traffic / minb <= 1.5) if traffic else None}

    materialized = None
    sp_bytes = w.B * w.Hq * w.N * w.N * (4 + w.elem_bytes)
    if not w.materialized and not args.no_materialized and not fp8:
        materialized = {"skipped": f"S and P would take {sp_bytes / 1e9:.1f} GB; this workload "
                                   "runs only the tiled path (long_b4_h32_n4096_d128, "
                                   "gpt2_medium_b64_h16_n1024_d64 and the sequence-length "
                                   "sweep up to N = 8192 carry the comparison)"}
    elif not args.no_materialized and not fp8 and sp_bytes < (64 << 30):
        s = torch.empty((w.B, w.Hq, w.N, w.N), dtype=torch.float32, device="cuda")
        p = torch.empty((w.B, w.Hq, w.N, w.N), dtype=w.torch_dtype, device="cuda")
        o2 = torch.empty_like(qd)
        l2 = torch.empty_like(lse)
        ment = attn.attn_fwd_materialized if w.dtype == "bf16" else attn.attn_fwd_materialized_f32

        def mstep():
            ment(qd, kd, vd, o2, l2, s, p, scale, stream)

        with torch.cuda.stream(stream):
            m_ms, m_ev, _, _ = time_launches(mstep, stream, max(3, args.steps // 5), 2)
        pred = acc.materialized_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, w.elem_bytes)
        meas = materialized_traffic_from_profiles(w.name)
        mbytes = sum(meas) if meas else None
        materialized = {"ms": round(m_ev, 4), "tflops": round(flops / (m_ev * 1e-3) / 1e12, 2),
                        "predicted_bytes": pred, "predicted_vs_min": round(pred / minb, 2),
                        "measured_bytes": mbytes,
                        "measured_read_write": list(meas) if meas else None,
                        "measured_vs_predicted": round(mbytes / pred, 3) if mbytes else None,
                        "measured_vs_min": round(mbytes / minb, 2) if mbytes else None,
                        "hbm_gbps": round(mbytes / (m_ev * 1e-3) / 1e9, 1) if mbytes else None,
                        "hbm_frac": (round(mbytes / (m_ev * 1e-3) / 1e9 / acc.PEAK_HBM_GBPS, 4)
                                     if mbytes else None),
                        "speedup_fused": round(m_ev / ev_mean, 2)}
        del s, p

    backward = None
    if args.backward and w.dtype == "bf16":
        g = torch.Generator().manual_seed(w.seed + 9)
        dout = torch.randn(qd.shape, generator=g).to(torch.bfloat16).cuda()
        o_f, lse_f = attn.fwd(qd, kd, vd, scale)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        ws_b = torch.empty(attn.attn_bwd_workspace_bytes(w.B, w.Hq, w.N), dtype=torch.uint8,
                           device="cuda")

        def bstep():
            attn.attn_bwd(qd, kd, vd, o_f, lse_f, dout, dq, dk, dv, ws_b, scale, stream)

        with torch.cuda.stream(stream):
            _, b_ms, _, _ = time_launches(bstep, stream, max(5, args.steps // 2), 3)
        # the usual accounting: 5 N x N x d products = 2.5x the forward's FLOPs
        # (the kernels run 7: S and dP are computed by both the dK/dV and
        # the dQ kernel)
        b_tflops = 2.5 * flops / (b_ms * 1e-3) / 1e12
        b_min = acc.bwd_min_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, w.elem_bytes)
        b_meas = backward_traffic_from_profiles(w.name)
        b_bytes = sum(b_meas) if b_meas else None
        backward = {"ms": round(b_ms, 4), "tflops": round(b_tflops, 2),
                    "frac": round(b_tflops / peak, 4),
                    "flops": "2.5 x forward (5 products)",
                    "executed_flops": "3.5 x forward (7 products)",
                    "min_bytes": b_min, "measured_bytes": b_bytes,
                    "measured_read_write": list(b_meas) if b_meas else None,
                    "measured_vs_min": round(b_bytes / b_min, 2) if b_bytes else None,
                    "hbm_gbps": round(b_bytes / (b_ms * 1e-3) / 1e9, 1) if b_bytes else None,
                    "fwd_plus_bwd_ms": round(b_ms + ev_mean, 4)}
        del dout, o_f, lse_f, dq, dk, dv, ws_b

    ceiling = None
    if not args.no_ceiling and w.dtype == "bf16" and not fp8:
        qz, kz, vz = torch.zeros_like(qd), torch.zeros_like(kd), torch.zeros_like(vd)
        ceiling = mfma_ceiling(lambda: entry(qz, kz, vz, o, lse, scale, stream), stream, flops,
                               args.steps)
        ceiling["attn_frac_of_gemm"] = round(achieved / ceiling["gemm_tflops"], 4)
        del qz, kz, vz

    cpu = None
    if not args.no_cpu_baseline:
        if fp8:
            # the 8-bit oracle is the plain definition on the dequantised inputs
            import oracle
            q, k, v = (torch.from_numpy(x) for x in oracle.dequantize(
                fp8[0].numpy(), fp8[1].numpy(), fp8[2].numpy(), *fp8[3:], w.N))
        cpu = cpu_baseline(w, q, k, v, scale, args.cpu_budget, args.cpu_threads)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "warmup_run": {"launches": n_warm, "ms": round(warm_ms, 1)},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else ("bf16" if w.dtype == "bf16" else "f32"),
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "io_dtype": "e4m3 in, bf16 out" if fp8 else w.dtype, "parallelism": "none",
                   "inputs": "iid N(0,1), seeded" + (", E4M3 with per-tensor scales" if fp8 else ""),
                   "entry": f"attn_fwd_split(n_split={args.split})" if args.split else
                            "attn_fwd_fp8" if fp8 else
                            ("attn_fwd" if w.dtype == "bf16" else "attn_fwd_f32")},
        "pct_peak": round(100 * value / peak, 2),
        "roofline": roofline,
        "materialized": materialized,
        "backward": backward,
        "mfma_ceiling": ceiling,
        "cpu_baseline": cpu,
        "kernel_source_sha": kernel_source_hash(w.name),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
