"""Summaries of rocprofv3 output for the committed profiles.

    python -m exact_io_aware_73_amd.profiling stats  <trace_kernel_stats.csv> <out.txt> "<command>"
        [<trace_kernel_trace.csv> <last_k>]
    python -m exact_io_aware_73_amd.profiling counters <workload> <fetch.csv> <write.csv>
        <copy_fetch.csv> <copy_write.csv> <copy_mib> <out.json> "<commands>" <kernel_source_sha>
        [<kernel>,<kernel>,...]
    python -m exact_io_aware_73_amd.profiling sq <out.txt> "<title and commands>" <kernel>
        <key tiles per wave> <pmc.csv> [<pmc.csv> ...]

``stats`` turns a ``--kernel-trace --stats`` CSV into a short text table;
given the per-dispatch trace and K, it adds each kernel's mean over its
last K dispatches (the timed steps of a bench run, after its warm-up).
``sq`` summarises SQ / GRBM counter runs of one kernel per wave-tile.
``counters`` turns two ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of
the fused kernel, and the same two counters read on a plain device copy of
known size, into HBM bytes per launch: each counter (KiB per dispatch) is
scaled by known copy bytes / the counter's reading on the copy.  Given a
comma-separated list of kernel names (substrings), the bytes of one call
are the sum over those kernels of each one's median dispatch (the
materialising path runs three kernels per call).
"""
from __future__ import annotations

import csv
import json
import statistics
import sys

FUSED_KERNEL = "attn_fwd_bf16_rows"
COPY_KERNEL = "copyBuffer"


def kernel_stats_table(path: str, command: str) -> str:
    rows = list(csv.DictReader(open(path)))
    lines = [f"command: {command}", "",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in rows:
        name = r["Name"]
        short = name if len(name) <= 60 else name[:57] + "..."
        lines.append(f"{short:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                     f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f} "
                     f"{float(r['Percentage']):6.2f}")
    lines.append("")
    lines.append("full kernel names:")
    lines += [f"  {r['Name']}" for r in rows]
    return "\n".join(lines) + "\n"


def last_k_table(trace_path: str, last_k: int) -> str:
    """Mean / min / max duration of each kernel's last `last_k` dispatches."""
    by_name = {}
    for r in csv.DictReader(open(trace_path)):
        by_name.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    lines = ["", f"last {last_k} dispatches of each kernel (the timed steps):",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}"]
    for name, ds in by_name.items():
        ds.sort()
        tail = [d for _, d in ds[-last_k:]]
        short = name if len(name) <= 60 else name[:57] + "..."
        lines.append(f"{short:60s} {len(tail):6d} {statistics.mean(tail) / 1e3:10.1f} "
                     f"{min(tail) / 1e3:10.1f} {max(tail) / 1e3:10.1f}")
    return "\n".join(lines) + "\n"


def counter_kib(path: str, kernel_substr: str):
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if kernel_substr in r["Kernel_Name"]]
    if not vals:
        raise ValueError(f"no dispatch of a kernel matching {kernel_substr!r} in {path}")
    return vals


def counters_summary(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_mib,
                     commands, kernel_source_sha, kernels=(FUSED_KERNEL,)):
    copy_bytes = int(copy_mib) << 20
    cf = statistics.median(counter_kib(copy_fetch_csv, COPY_KERNEL))
    cw = statistics.median(counter_kib(copy_write_csv, COPY_KERNEL))
    f_scale = copy_bytes / (cf * 1024)
    w_scale = copy_bytes / (cw * 1024)
    fetch = write = 0.0
    per_kernel = {}
    for kern in kernels:
        fk = counter_kib(fetch_csv, kern)
        wk = counter_kib(write_csv, kern)
        kf = statistics.median(fk) * 1024 * f_scale
        kw = statistics.median(wk) * 1024 * w_scale
        fetch += kf
        write += kw
        per_kernel[kern] = {"fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
                            "read_bytes": round(kf), "write_bytes": round(kw)}
    rec = {"workload": workload, "kernel": ",".join(kernels)}
    if len(kernels) == 1:
        rec.update({k: v for k, v in per_kernel[kernels[0]].items() if k.endswith("dispatch")})
    else:
        rec["per_kernel"] = per_kernel
    rec.update({
        "copy_probe_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
        "hbm_read_bytes_per_launch": round(fetch), "hbm_write_bytes_per_launch": round(write),
        "hbm_bytes_per_launch": round(fetch + write),
        "kernel_source_sha": kernel_source_sha, "commands": commands,
    })
    return rec


def sq_summary(csv_paths, kernel_substr: str, tiles_per_wave: int, n_simd: int = 1024,
               n_xcd: int = 8) -> dict:
    """Per-dispatch SQ / GRBM counters of one kernel (summed over the
    counter instances), the dispatch duration, and figures per wave-tile
    (one wave's pass over one key tile): instructions by kind, the matrix-
    core and vector-ALU busy cycles, their overlap, and the clock
    (GRBM_GUI_ACTIVE per XCD over the dispatch time).  Cycle counters that
    count in units of four cycles (SQ_ACTIVE_INST_*, SQ_WAIT_*, SQ_WAVE_CYCLES)
    are scaled by 4."""
    per = {}
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            if kernel_substr not in r["Kernel_Name"]:
                continue
            d = per.setdefault((path, int(r["Dispatch_Id"])), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            d["_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            d["_name"] = r["Kernel_Name"]
    if not per:
        raise ValueError(f"no dispatch of {kernel_substr!r}")
    merged = {}
    for (path, _), d in per.items():
        for k, v in d.items():
            merged.setdefault(k, []).append(v)
    med = {k: statistics.median(v) for k, v in merged.items() if k != "_name"}
    waves = med.get("SQ_WAVES")
    out = {"kernel": merged["_name"][0], "dispatches": len(merged["_ns"]), "median": med}
    if waves:
        wt = waves * tiles_per_wave
        q4 = {"SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY",
              "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"}
        out["per_wave_tile"] = {k: round(v * (4 if k in q4 else 1) / wt, 1) for k, v in med.items()
                                if k.startswith("SQ_") and k != "SQ_WAVES"}
    if "GRBM_GUI_ACTIVE" in med:
        cyc = med["GRBM_GUI_ACTIVE"] / n_xcd
        out["clock_ghz"] = round(cyc / med["_ns"], 3)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            out["mfma_busy"] = round(med["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * n_simd), 3)
        if "SQ_ACTIVE_INST_VALU" in med:
            out["valu_busy"] = round(4 * med["SQ_ACTIVE_INST_VALU"] / (cyc * n_simd), 3)
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in med:
            out["mfma_valu_coexec"] = round(med["SQ_VALU_MFMA_COEXEC_CYCLES"] / (cyc * n_simd), 3)
    return out


def main(argv):
    if argv[0] == "stats":
        src, out, cmd = argv[1:4]
        text = kernel_stats_table(src, cmd)
        if len(argv) > 4:
            text += last_k_table(argv[4], int(argv[5]))
        open(out, "w").write(text)
    elif argv[0] == "counters":
        _, wl, f, w, cf, cw, mib, out, cmds, sha = argv[:10]
        kernels = tuple(argv[10].split(",")) if len(argv) > 10 else (FUSED_KERNEL,)
        rec = counters_summary(wl, f, w, cf, cw, int(mib), cmds, sha, kernels)
        json.dump(rec, open(out, "w"), indent=1)
        print(json.dumps({k: rec[k] for k in ("workload", "hbm_read_bytes_per_launch",
                                               "hbm_write_bytes_per_launch")}))
    elif argv[0] == "sq":
        out, title, kern, tiles = argv[1:5]
        rec = sq_summary(argv[5:], kern, int(tiles))
        with open(out, "w") as f:
            f.write(title.rstrip() + "\n\n" + json.dumps(rec, indent=1) + "\n")
        print(json.dumps({k: rec[k] for k in rec if k not in ("median", "per_wave_tile")}))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
