#!/usr/bin/env python3
"""Benchmark of block-sparse attention with routing and residual on one MI355X.

One step = the whole hot path on one attention layer: routing (pool, proxy,
select, schedule) followed by the sparse forward with the dropped-block
residual.  Inputs are seeded synthetic Q/K/V with the token-grid shape of the
workload, resident in HBM before the timed region.

    python bench.py [--steps K] [--warmup W] [--workload stress] [--tau-mode relative]

The default workload is the largest single-GPU layer shape: the stress case,
B = 2, H = 24, N = 118800 (a 33 x 45 x 80 token grid), d = 128, bf16, 128 x 128
blocks, tau = 0.05 relative, per-head query scales drawn from [1, 12].

Prints one JSON line.  value = dense-equivalent TFLOP/s = 4 B H N^2 d / step
time.  roofline: the forward kernel's algorithmic flops per launch (exact
kept tiles + one residual column per dropped block) over its average launch
time measured with HIP events on its stream, against the bf16 dense MFMA peak.
route: the routing kernels' algorithmic bytes (q, k, v read once; pooled key
and value means written in fp32 and bf16; kept-block indices and the bit mask
written) over their time, against the HBM peak.
cpu_baseline: the fp64 CPU oracle timed on a bounded sample of the same
workload and extrapolated in executed query-key pairs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dense-equiv TFLOP/s & ms/call per attention layer at 1 MI355X; MFMA % of peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
FLASH_SRC = os.path.join(ROOT, "free_block_sparse_route_amd", "csrc", "sa_flash.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="stress")
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--tau-mode", choices=("relative", "absolute", "topp"), default="relative")
    ap.add_argument("--sparsepr", type=int, default=0, metavar="P",
                    help="also time the probe-fitted residual correction with P probes per query block and "
                         "compare its error against dense attention with the block residual's")
    ap.add_argument("--fused", action="store_true",
                    help="fused routing: the route pre-pass writes row statistics only and the forward "
                         "takes the keep decisions itself")
    ap.add_argument("--proxy", choices=("centroid", "pama"), default="centroid",
                    help="routing proxy: block means (default) or per-query block attention averaged per block")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--with-copy", action="store_true",
                    help="after the bench, run a plain 1 GiB device copy twice (scale of the HBM counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/flash_<workload>_<tau-mode>_traffic.{json,md} from the counter "
                         "collections of two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of this "
                         "script with --with-copy, then exit")
    ap.add_argument("--mfma-summary", metavar="CSV",
                    help="write profiles/flash_<workload>_<tau-mode>_mfma.{json,md} from the counter collection "
                         "of a rocprofv3 --pmc run of this script (SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                         "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE) and its kernel trace "
                         "(KERNEL_TRACE_CSV, for the durations), then exit")
    ap.add_argument("--trace-csv", metavar="KERNEL_TRACE_CSV", help="kernel trace of the --mfma-summary run")
    ap.add_argument("--stats-summary", metavar="KERNEL_STATS_CSV",
                    help="write profiles/flash_<workload>_<tau-mode>_kernel_stats.md from the kernel_stats.csv of a "
                         "rocprofv3 --kernel-trace --stats run of this script (the library's kernels under the "
                         "profiler's own names), then exit")
    ap.add_argument("--sq-summary", nargs="+", metavar="CSV",
                    help="write profiles/route_<workload>_<tau-mode>_sq.md from the counter collections of "
                         "rocprofv3 --pmc passes over this script (SQ_* and GRBM_GUI_ACTIVE counters, one or more "
                         "passes) with --trace-csv for the durations: per kernel, the counters' means and the "
                         "issue and wait fractions they give, then exit")
    ap.add_argument("--pmc-command", default="", help="the command the counter runs used (recorded)")
    ap.add_argument("--no-residual-timing", action="store_true",
                    help="skip timing the forward without the residual fold (its share of the forward)")
    ap.add_argument("--cold-calls", type=int, default=20,
                    help="calls timed one by one after flushing the caches with a 512 MiB write (0: skip)")
    return ap.parse_args()


def source_hash() -> str:
    return hashlib.sha256(open(FLASH_SRC, "rb").read()).hexdigest()[:16]


def load_traffic(workload: str, tau_mode: str):
    """HBM bytes per forward launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"flash_{workload}_{tau_mode}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("flash_source_sha256_16") != source_hash():
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 1 << 30


def copy_calibration():
    """A plain device copy of COPY_BYTES (reads and writes that many bytes), twice."""
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()


def _pmc_rows(path: str, counter: str):
    import csv
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    if not rows:
        raise SystemExit(f"{path}: no {counter} rows")
    return rows


def _mean_kib(rows, pred):
    vals = [float(r["Counter_Value"]) for r in rows if pred(r)]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def pmc_summary(args):
    """HBM traffic of the sparse forward kernel per launch from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads for
    the plain 1 GiB copy in the same run."""
    fetch_rows = _pmc_rows(args.pmc_summary[0], "FETCH_SIZE")
    write_rows = _pmc_rows(args.pmc_summary[1], "WRITE_SIZE")
    is_flash = lambda r: "flash_kernel" in r["Kernel_Name"] and "Lb1ELb0E" in r["Kernel_Name"]
    # the copy: the dispatch of a kernel named for copying whose counter is the largest
    def copy_kib(rows):
        cands = [float(r["Counter_Value"]) for r in rows if "copy" in r["Kernel_Name"].lower()]
        if not cands:
            raise SystemExit("no copy dispatch in the counter collection (run with --with-copy)")
        return max(cands)
    f_kib, nf = _mean_kib(fetch_rows, is_flash)
    w_kib, nw = _mean_kib(write_rows, is_flash)
    if not nf or not nw:
        raise SystemExit("no sparse flash_kernel dispatch in the counter collections")
    copy_f, copy_w = copy_kib(fetch_rows), copy_kib(write_rows)
    scale_f = COPY_BYTES / (copy_f * 1024.0)
    scale_w = COPY_BYTES / (copy_w * 1024.0)
    rd = f_kib * 1024.0 * scale_f
    wr = w_kib * 1024.0 * scale_w
    rec = {"kernel": "flash_kernel (sparse forward with residual)", "workload": args.workload,
           "tau_mode": args.tau_mode, "proxy": args.proxy, "fused": args.fused, "flash_source_sha256_16": source_hash(),
           "bytes_per_launch": rd + wr, "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
           "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "dispatches": [nf, nw],
           "copy_fetch_kib": copy_f, "copy_write_kib": copy_w, "fetch_scale": scale_f, "write_scale": scale_w,
           "command": args.pmc_command}
    # every kernel of the run, by the same scales (the routing kernels among them)
    per_kernel = []
    for name in sorted({r["Kernel_Name"] for r in fetch_rows} | {r["Kernel_Name"] for r in write_rows}):
        fk, n1 = _mean_kib(fetch_rows, lambda r, n=name: r["Kernel_Name"] == n)
        wk, n2 = _mean_kib(write_rows, lambda r, n=name: r["Kernel_Name"] == n)
        per_kernel.append({"kernel": _short_kernel(name), "kernel_name": name, "dispatches": [n1, n2],
                           "read_bytes_per_launch": None if fk is None else fk * 1024.0 * scale_f,
                           "write_bytes_per_launch": None if wk is None else wk * 1024.0 * scale_w})
    rec["all_kernels"] = per_kernel
    base = os.path.join(ROOT, "profiles", f"flash_{args.workload}_{args.tau_mode}_traffic")
    with open(base + ".json", "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    with open(base + ".md", "w") as f:
        f.write(f"# HBM traffic of the sparse forward kernel: {args.workload}, {args.tau_mode} tau\n\n")
        f.write("Counter runs (one counter per pass, each over the same command):\n\n")
        f.write(f"    {args.pmc_command}\n\n")
        f.write("| quantity | value |\n|---|---|\n")
        f.write(f"| FETCH_SIZE per flash dispatch | {f_kib:,.0f} KiB (mean of {nf}) |\n")
        f.write(f"| WRITE_SIZE per flash dispatch | {w_kib:,.0f} KiB (mean of {nw}) |\n")
        f.write(f"| FETCH_SIZE of the 1 GiB copy | {copy_f:,.0f} KiB -> scale {scale_f:.4f} |\n")
        f.write(f"| WRITE_SIZE of the 1 GiB copy | {copy_w:,.0f} KiB -> scale {scale_w:.4f} |\n")
        f.write(f"| read bytes per launch (scaled) | {rd / 1e9:.3f} GB |\n")
        f.write(f"| written bytes per launch (scaled) | {wr / 1e9:.3f} GB |\n")
        f.write(f"| kernel source sha256[:16] | {rec['flash_source_sha256_16']} |\n")
        f.write("\nEvery kernel of the run, by the same scales (bytes per launch):\n\n")
        f.write("| kernel | dispatches | read MB | written MB |\n|---|---|---|---|\n")
        mb = lambda x: "-" if x is None else f"{x / 1e6:,.1f}"
        for r in per_kernel:
            f.write(f"| {r['kernel']} | {r['dispatches'][0]} | {mb(r['read_bytes_per_launch'])} | "
                    f"{mb(r['write_bytes_per_launch'])} |\n")
    print(json.dumps(rec))


def _short_kernel(name: str) -> str:
    """Readable label of a rocprof kernel name (the full name is kept beside it)."""
    if "flash_kernel" in name:
        dt = "bf16" if "DF16b" in name else "f32"
        kind = "fused" if "Lb1ELb1E" in name else ("sparse" if "Lb1ELb0E" in name else "dense")
        return f"flash_kernel {dt} {kind}"
    for k in ("pool_kernel", "select_kernel", "order_kernel", "pama_kernel", "permute_kernel"):
        if k in name:
            return k
    return name[:60]


def mfma_summary(args):
    """Matrix-core counters per kernel from one rocprofv3 --pmc pass
    (SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES,
    GRBM_GUI_ACTIVE) with the kernel trace of the same run (durations):
      MFMA flops per launch = MOPS_BF16 x 512 (the counter's unit),
      MFMA busy = sum of SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs),
      shader clock = GRBM_GUI_ACTIVE / kernel duration."""
    import csv
    rows = list(csv.DictReader(open(args.mfma_summary)))
    # the profiler reports GRBM_GUI_ACTIVE summed over the dies (one GRBM each)
    # and SQ counters summed over every SIMD; the agent table gives both counts
    n_xcc, simds = 8, 256 * 4
    info = os.path.join(os.path.dirname(args.mfma_summary), os.path.basename(args.mfma_summary).replace(
        "counter_collection", "agent_info"))
    if os.path.exists(info):
        for r in csv.DictReader(open(info)):
            if r.get("Name", "").startswith("gfx"):
                n_xcc, simds = int(r["Num_Xcc"]), int(r["Simd_Count"])
    dur = {}
    if args.trace_csv:
        for r in csv.DictReader(open(args.trace_csv)):
            dur[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    per = {}
    for r in rows:
        d = per.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"]})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    kernels = {}
    for did, d in per.items():
        k = kernels.setdefault(d["name"], [])
        d["dur_s"] = dur.get(did)
        k.append(d)
    out = []
    for name, ds in kernels.items():
        mean = lambda key: sum(x.get(key, 0.0) for x in ds) / len(ds)
        flops = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512.0
        grbm = mean("GRBM_GUI_ACTIVE") / n_xcc        # busy cycles of the GPU clock
        busy = mean("SQ_VALU_MFMA_BUSY_CYCLES")
        durs = [x["dur_s"] for x in ds if x["dur_s"]]
        t = sum(durs) / len(durs) if durs else None
        rec = {"kernel": _short_kernel(name), "kernel_name": name, "dispatches": len(ds),
               "mfma_bf16_flops_per_launch": flops, "mfma_busy_frac": busy / (grbm * simds) if grbm else None,
               "grbm_gui_active": grbm, "sq_busy_cycles": mean("SQ_BUSY_CYCLES"),
               "avg_duration_ms": t * 1e3 if t else None,
               "clock_ghz": grbm / t / 1e9 if t and grbm else None,
               "mfma_bf16_tflops": flops / t / 1e12 if t else None,
               "mfma_bf16_frac_of_peak": flops / t / 1e12 / PEAK_BF16_TFLOPS if t else None}
        out.append(rec)
    out.sort(key=lambda r: -(r["avg_duration_ms"] or 0) * r["dispatches"])
    rec = {"workload": args.workload, "tau_mode": args.tau_mode, "flash_source_sha256_16": source_hash(),
           "kernels": out, "command": args.pmc_command}
    base = os.path.join(ROOT, "profiles", f"flash_{args.workload}_{args.tau_mode}_mfma")
    with open(base + ".json", "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    with open(base + ".md", "w") as f:
        f.write(f"# Matrix-core counters: {args.workload}, {args.tau_mode} tau\n\n")
        f.write("One rocprofv3 counter pass with the kernel trace (durations), then the summary:\n\n")
        f.write(f"    {args.pmc_command}\n\n")
        f.write("MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; GPU cycles = GRBM_GUI_ACTIVE / 8 (the "
                "profiler sums it over the 8 dies); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GPU cycles x 1024 "
                "SIMDs); clock = GPU cycles / duration (the kernel runs alone under counter collection).\n\n")
        f.write("| kernel | dispatches | avg ms | MFMA bf16 GFLOP per launch | MFMA TFLOP/s | frac of 2500 | "
                "MFMA busy | clock GHz |\n|---|---|---|---|---|---|---|---|\n")
        fmt = lambda x, spec: "-" if x is None else format(x, spec)
        for r in out:
            f.write(f"| {r['kernel']} | {r['dispatches']} | {fmt(r['avg_duration_ms'], '.3f')} | "
                    f"{r['mfma_bf16_flops_per_launch'] / 1e9:,.1f} | {fmt(r['mfma_bf16_tflops'], ',.0f')} | "
                    f"{fmt(r['mfma_bf16_frac_of_peak'], '.3f')} | {fmt(r['mfma_busy_frac'], '.3f')} | "
                    f"{fmt(r['clock_ghz'], '.2f')} |\n")
        f.write(f"\nKernel source sha256[:16] (sa_flash.hip): {rec['flash_source_sha256_16']}\n")
    print(json.dumps(rec))


def stats_summary(args):
    """The library's kernels from a rocprofv3 --kernel-trace --stats table, under
    the names the profiler prints."""
    import csv
    rows = [r for r in csv.DictReader(open(args.stats_summary))
            if any(k in r["Name"] for k in ("flash_kernel", "pool_kernel", "select_kernel", "order_",
                                             "pama_kernel", "permute_kernel", "pr_", "probe_gather"))]
    path = os.path.join(ROOT, "profiles", f"flash_{args.workload}_{args.tau_mode}_kernel_stats.md")
    with open(path, "w") as f:
        f.write(f"# Kernel times: {args.workload}, {args.tau_mode} tau\n\n")
        f.write("rocprofv3 kernel trace with per-kernel statistics (kernel_stats.csv, the library's rows):\n\n")
        f.write(f"    {args.pmc_command}\n\n")
        f.write("| kernel (as rocprofv3 names it) | calls | avg us | min us | max us | % of GPU time |\n"
                "|---|---|---|---|---|---|\n")
        for r in rows:
            f.write(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:,.1f} | "
                    f"{float(r['MinNs']) / 1e3:,.1f} | {float(r['MaxNs']) / 1e3:,.1f} | {float(r['Percentage']):.2f} |\n")
        f.write(f"\nKernel source sha256[:16] (sa_flash.hip): {source_hash()}\n")
    print(path)


def sq_summary(args):
    """Per-kernel SQ counters from one or more rocprofv3 --pmc passes of this
    script.  The wave counters (SQ_WAVE_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY,
    SQ_ACTIVE_INST_*) count in units of four cycles; their ratios to
    SQ_WAVE_CYCLES are the fractions of a wave's lifetime.  Resident waves per
    CU = 4 SQ_WAVE_CYCLES / (GPU cycles x CUs); GPU cycles = GRBM_GUI_ACTIVE /
    dies (the profiler sums it over the dies); MFMA busy as in --mfma-summary."""
    import csv
    n_xcc, simds, cus = 8, 256 * 4, 256
    dur = {}
    if args.trace_csv:
        for r in csv.DictReader(open(args.trace_csv)):
            dur.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    vals = {}
    for path in args.sq_summary:
        info = os.path.join(os.path.dirname(path), os.path.basename(path).replace("counter_collection", "agent_info"))
        if os.path.exists(info):
            for r in csv.DictReader(open(info)):
                if r.get("Name", "").startswith("gfx"):
                    n_xcc, simds, cus = int(r["Num_Xcc"]), int(r["Simd_Count"]), int(r["Cu_Count"])
        per = {}
        for r in csv.DictReader(open(path)):
            d = per.setdefault((r["Dispatch_Id"], r["Kernel_Name"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for (_, name), d in per.items():
            k = vals.setdefault(name, {})
            for c, x in d.items():
                k.setdefault(c, []).append(x)
    lib = ("flash_kernel", "pool_kernel", "select_kernel", "order", "pama_kernel", "permute_kernel")
    path = os.path.join(ROOT, "profiles", f"route_{args.workload}_{args.tau_mode}_sq.md")
    with open(path, "w") as f:
        f.write(f"# SQ counters of the library's kernels: {args.workload}, {args.tau_mode} tau\n\n")
        f.write("rocprofv3 --pmc passes (each a separate run of the same command), with the kernel trace of a "
                "run for the durations:\n\n")
        f.write(f"    {args.pmc_command}\n\n")
        f.write("Wave counters count in units of four cycles. Fractions are of SQ_WAVE_CYCLES (the waves' "
                "lifetime): waiting to issue (SQ_WAIT_INST_ANY), waiting on a counter (SQ_WAIT_ANY, memory and "
                "LDS), issuing (SQ_ACTIVE_INST_ANY). Resident waves per CU = 4 SQ_WAVE_CYCLES / (GPU cycles x "
                f"{cus} CUs); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GPU cycles x {simds} SIMDs); VALU busy = 4 "
                f"SQ_ACTIVE_INST_VALU / (GPU cycles x {simds} SIMDs) (a wave-64 VALU instruction holds its SIMD "
                "four cycles).\n\n")
        f.write("| kernel | avg us | clock GHz | waves | resident waves / CU | wait to issue | wait on counter | "
                "issuing | MFMA busy | VALU busy | VALU / wave | SALU / wave | LDS / wave |\n"
                "|---|---|---|---|---|---|---|---|---|---|---|---|---|\n")
        mean = lambda d, c: (sum(d[c]) / len(d[c])) if c in d else None
        for name, d in vals.items():
            if not any(k in name for k in lib):
                continue
            t = dur.get(name)
            t = sorted(t)[len(t) // 2] if t else None
            grbm = mean(d, "GRBM_GUI_ACTIVE")
            cyc = grbm / n_xcc if grbm else None
            wc = mean(d, "SQ_WAVE_CYCLES")
            waves = mean(d, "SQ_WAVES")
            frac = lambda c: "-" if wc is None or c not in d else f"{mean(d, c) / wc:.2f}"
            per_wave = lambda c: "-" if waves is None or c not in d else f"{mean(d, c) / waves:,.0f}"
            res = f"{4 * wc / (cyc * cus):.1f}" if wc and cyc else "-"
            mb = f"{mean(d, 'SQ_VALU_MFMA_BUSY_CYCLES') / (cyc * simds):.2f}" if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in d else "-"
            vb = f"{4 * mean(d, 'SQ_ACTIVE_INST_VALU') / (cyc * simds):.2f}" if cyc and "SQ_ACTIVE_INST_VALU" in d else "-"
            f.write(f"| {_short_kernel(name)} | {'-' if t is None else f'{t * 1e6:,.1f}'} | "
                    f"{'-' if not (t and cyc) else f'{cyc / t / 1e9:.2f}'} | {'-' if waves is None else f'{waves:,.0f}'} | "
                    f"{res} | {frac('SQ_WAIT_INST_ANY')} | {frac('SQ_WAIT_ANY')} | {frac('SQ_ACTIVE_INST_ANY')} | "
                    f"{mb} | {vb} | {per_wave('SQ_INSTS_VALU')} | {per_wave('SQ_INSTS_SALU')} | {per_wave('SQ_INSTS_LDS')} |\n")
        f.write("\nMeans per dispatch of every counter:\n\n| kernel | counter | mean | dispatches |\n|---|---|---|---|\n")
        for name, d in vals.items():
            if not any(k in name for k in lib):
                continue
            for c in sorted(d):
                f.write(f"| {_short_kernel(name)} | {c} | {mean(d, c):,.0f} | {len(d[c])} |\n")
    print(path)


def load_mfma(workload: str, tau_mode: str):
    """The sparse forward's matrix-core counters from the committed summary, if taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"flash_{workload}_{tau_mode}_mfma.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("flash_source_sha256_16") != source_hash():
        return None
    for r in rec["kernels"]:
        if r["kernel"].startswith("flash_kernel") and r["kernel"].endswith("sparse"):
            return {k: r[k] for k in ("mfma_bf16_flops_per_launch", "mfma_busy_frac", "clock_ghz",
                                      "mfma_bf16_frac_of_peak", "avg_duration_ms")}
    return None


def cpu_baseline(w, cfg, Qc, Kc, Vc, budget_s: float = 12.0):
    """The oracle as it stands, on the host cores: routing of every head in full,
    outputs on a seeded sample of query blocks until about budget_s seconds of
    forward work, extrapolated linearly in executed query-key pairs."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import sparse_attn_ref as R

    cores = len(os.sched_getaffinity(0))
    p = R.RouteParams(cfg.block_q, cfg.block_k, float(np.float32(cfg.tau)), cfg.tau_mode, cfg.max_keep,
                      cfg.min_keep, cfg.n_dense_prefix, cfg.scale)
    n_j = R.block_counts(w.N, w.block_k)
    m_i = R.block_counts(w.N, w.block_q)
    with threadpool_limits(limits=cores):
        used = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
        t0 = time.perf_counter()
        heads = {}
        for b in range(w.B):
            for h in range(w.H):
                q = Qc[b, h].double().numpy()
                k = Kc[b, h].double().numpy()
                heads[(b, h)] = R.route_ref(q, k, p).mask
        t_route = time.perf_counter() - t0

        def pairs(mask_row, I):
            return int(m_i[I]) * (int((n_j * mask_row).sum()) + int((~mask_row).sum()))

        total_pairs = sum(pairs(m[I], I) for m in heads.values() for I in range(m.shape[0]))
        rng = np.random.default_rng(0)
        order = [(bh, int(I)) for bh in heads for I in range(w.n_qb)]
        rng.shuffle(order)
        t_fwd = 0.0
        done_pairs = 0
        n_blocks = 0
        cache = {}
        for (b, h), I in order:
            if (b, h) not in cache:
                cache.clear()
                cache[(b, h)] = tuple(T[b, h].double().numpy() for T in (Qc, Kc, Vc))
            q, k, v = cache[(b, h)]
            t1 = time.perf_counter()
            R.forward_ref_with_mask(q, k, v, heads[(b, h)], p, rows=[I])
            t_fwd += time.perf_counter() - t1
            done_pairs += pairs(heads[(b, h)][I], I)
            n_blocks += 1
            if t_fwd >= budget_s:
                break
    t_total = t_route + t_fwd * total_pairs / max(done_pairs, 1)
    dense = 4.0 * w.B * w.H * w.N * w.N * w.d
    return {"value": dense / t_total / 1e12, "unit": "TFLOP/s", "cores": int(used), "kind": "oracle",
            "sample": (f"routing of all {len(heads)} heads timed in full ({t_route:.1f} s); forward on "
                       f"{n_blocks} random query blocks ({t_fwd:.1f} s, {done_pairs / total_pairs:.2%} of the "
                       f"executed query-key pairs), extrapolated linearly in executed pairs"),
            "ms_per_step_extrapolated": t_total * 1e3, "host_cores_visible": cores}


def median(xs):
    xs = sorted(xs)
    k = len(xs)
    return 0.5 * (xs[(k - 1) // 2] + xs[k // 2])


FLUSH_BYTES = 512 << 20


def cold_timing(sa, Q, K, V, rt, O, cfg, calls):
    """Median route and forward times with cold caches: before each call a 512 MiB
    buffer is written, which evicts the inputs from the L2s and the 256 MB
    Infinity Cache.  The write is outside the timed events."""
    import torch
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    r_ms, f_ms = [], []
    for i in range(calls):
        flush.fill_(float(i))
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        sa.route(Q, K, V, cfg, out=rt)
        e[1].record()
        flush.fill_(float(i) + 0.5)            # the forward, too, starts cold
        e2 = torch.cuda.Event(enable_timing=True)
        e2.record()
        sa.forward(Q, K, V, rt, cfg, out=O)
        e[2].record()
        torch.cuda.synchronize()
        r_ms.append(e[0].elapsed_time(e[1]))
        f_ms.append(e2.elapsed_time(e[2]))
    del flush
    return {"route_ms_median": median(r_ms), "forward_ms_median": median(f_ms), "calls": calls,
            "flush_bytes": FLUSH_BYTES}


def stream_copy_rate(reps=10):
    """A STREAM-like device copy: median GB/s of copying COPY_BYTES, counting the
    bytes read and the bytes written; the measured reference for the routing's
    HBM-bound pass beside the published peak."""
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del a, b
    return 2.0 * COPY_BYTES / (median(ts) * 1e-3) / 1e9


def permute_timing(sa, X, w, reps=10):
    """Token reordering of one [B, H, N, d] tensor into the workload's Hilbert
    order (gather) and back (scatter): median ms and GB/s, counting every row
    read once and written once."""
    import torch
    perm = sa.hilbert_order(*w.grid).cuda()
    Y = torch.empty_like(X)
    Z = torch.empty_like(X)
    res = {}
    for name, src, dst, inv in (("gather", X, Y, False), ("scatter", Y, Z, True)):
        sa.permute_tokens(src, perm, w.n_text, inverse=inv, out=dst)
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            sa.permute_tokens(src, perm, w.n_text, inverse=inv, out=dst)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = median(ts)
        gbs = 2.0 * X.numel() * X.element_size() / (ms * 1e-3) / 1e9
        res[name] = {"ms_median": ms, "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS}
    torch.cuda.synchronize()
    assert torch.equal(Z, X), "permutation round trip"
    return res


def sparsepr_compare(sa, Q, K, V, rt, cfg, O, P, rank=8, ridge=1e-3, reps=5):
    """Median time of the probe-fitted correction (P probes per query block) and the
    relative Frobenius error against the library's dense path of: the forward
    with the block residual, the probe-fitted output, the kept tokens alone."""
    import dataclasses
    import torch
    ws = torch.empty(sa.sparsepr_workspace_size(Q, cfg, P), dtype=torch.uint8, device=Q.device)
    Opr = torch.empty_like(O)
    ts = []
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sa.forward_sparsepr(Q, K, V, rt, cfg, probes_per_block=P, rank=rank, ridge=ridge, out=Opr, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    Okept = sa.forward(Q, K, V, rt, dataclasses.replace(cfg, no_residual=True))
    Od = sa.dense_ref_gpu(Q, K, V, block_q=cfg.block_q)
    torch.cuda.synchronize()
    err = lambda A: float(torch.linalg.norm((A.float() - Od.float()).flatten()) / torch.linalg.norm(Od.float().flatten()))
    return {"probes_per_block": P, "rank": rank, "ridge": ridge, "ms_median": median(ts[1:]),
            "rel_fro_vs_dense": {"block_residual": err(O), "probe_fitted": err(Opr), "kept_tokens_only": err(Okept)}}


def issued_mfma_flops(w, rt, mask, cfg):
    """Matrix-core flops the forward kernel issues per launch, counting padded
    rows: every query block runs block_q rows (the last one padded), every kept
    key block ceil(n_J / rows) exact tiles of `rows` keys (padded), and every
    group of 32 pooled blocks with a dropped one a residual tile.  Per wave
    (32 query rows) a tile takes, in 32x32x16 bf16 MFMAs of 32768 flops:
    bf16 exact d/4; bf16 residual 3d/16 (the value remainders are not read);
    fp32 exact or residual 5d/16 (split products)."""
    import torch
    d = w.d
    rows = 64 if w.dtype == "bf16" else 32
    n_j = torch.tensor([min(w.block_k, w.N - J * w.block_k) for J in range(rt.n_kb)], device=mask.device,
                       dtype=torch.int64)
    tiles_j = (n_j + rows - 1) // rows
    exact_tiles = int((mask.long() * tiles_j).sum())
    words = -(-rt.n_kb // 32)
    pad = words * 32 - rt.n_kb
    dropped = ~mask
    if pad:
        dropped = torch.nn.functional.pad(dropped, (0, pad), value=False)
    resid_tiles = int(dropped.view(*dropped.shape[:-1], words, 32).any(-1).sum())
    if cfg.no_residual:
        resid_tiles = 0
    per_exact = d // 4 if w.dtype == "bf16" else 5 * d // 16
    per_resid = 3 * d // 16 if w.dtype == "bf16" else 5 * d // 16
    waves = w.block_q // 32
    return float((exact_tiles * per_exact + resid_tiles * per_resid) * waves * 32768)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not supported: "
              "heads shard across GPUs with no exchange inside attention, so the per-GPU kernel "
              "measured at --gpus 1 is the figure of interest.", file=sys.stderr)
        sys.exit(2)
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.mfma_summary:
        mfma_summary(args)
        return
    if args.stats_summary:
        stats_summary(args)
        return
    if args.sq_summary:
        sq_summary(args)
        return

    import torch

    import free_block_sparse_route_amd as sa
    from workloads import synth as S

    w = S.WORKLOADS[args.workload]
    mode = {"relative": sa.RELATIVE, "absolute": sa.ABSOLUTE, "topp": sa.TOPP}[args.tau_mode]
    cfg = sa.Config(block_q=w.block_q, block_k=w.block_k, tau=w.tau if args.tau is None else args.tau,
                    tau_mode=mode, max_keep=w.max_keep, min_keep=1, n_dense_prefix=w.n_text,
                    proxy=sa.PAMA if args.proxy == "pama" else sa.CENTROID, fused=args.fused)
    print(f"[bench] generating {w.name} B{w.B} H{w.H} N{w.N} d{w.d}", file=sys.stderr, flush=True)
    Qc, Kc, Vc = S.make_qkv(w)
    Q, K, V = Qc.cuda(), Kc.cuda(), Vc.cuda()
    rt = sa.route(Q, K, V, cfg)
    O = sa.forward(Q, K, V, rt, cfg)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        sa.route(Q, K, V, cfg, out=rt)
        sa.forward(Q, K, V, rt, cfg, out=O)
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        sa.route(Q, K, V, cfg, out=rt)
        ev[i][1].record()
        sa.forward(Q, K, V, rt, cfg, out=O)
        ev[i][2].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    route_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    fwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    warm = {"route_ms_median": median([e[0].elapsed_time(e[1]) for e in ev]),
            "forward_ms_median": median([e[1].elapsed_time(e[2]) for e in ev])}
    cold = cold_timing(sa, Q, K, V, rt, O, cfg, args.cold_calls) if args.cold_calls > 0 else None

    # algorithmic work of one forward launch, from the route it consumed
    mask = rt.mask()
    n_j = torch.tensor([min(w.block_k, w.N - J * w.block_k) for J in range(rt.n_kb)], device=mask.device,
                       dtype=torch.float64)
    m_i = torch.tensor([min(w.block_q, w.N - I * w.block_q) for I in range(rt.n_qb)], device=mask.device,
                       dtype=torch.float64)
    kept_tok = (mask.double() * n_j).sum(-1)                  # [B,H,n_qb]
    dropped = (~mask).double().sum(-1)
    exact_flops = float(4.0 * w.d * (m_i * kept_tok).sum())
    resid_flops = float(4.0 * w.d * (m_i * dropped).sum())
    dense_flops = 4.0 * w.B * w.H * w.N * w.N * w.d
    kept_frac = exact_flops / dense_flops
    issued = issued_mfma_flops(w, rt, mask, cfg)
    fwd_tflops = (exact_flops + resid_flops) / (fwd_ms * 1e-3) / 1e12

    es = 2 if w.dtype == "bf16" else 4
    words = -(-rt.n_kb // 32)
    route_read = 3.0 * w.B * w.H * w.N * w.d * es
    route_written = (2.0 * w.B * w.H * rt.n_kb * w.d * (4 + 2)       # key and value means, fp32 and bf16
                     + 4.0 * float(mask.sum())                       # kept-block indices
                     + 4.0 * w.B * w.H * rt.n_qb * words)            # bit mask
    route_bytes = route_read + route_written
    route_gbs = route_bytes / (route_ms * 1e-3) / 1e9
    stream_gbs = stream_copy_rate()

    # the forward without the residual fold, on the same route: the residual's share
    noresid = None
    if not args.no_residual_timing:
        import dataclasses
        cfg_nr = dataclasses.replace(cfg, no_residual=True)
        On = torch.empty_like(O)
        sa.forward(Q, K, V, rt, cfg_nr, out=On)
        ts = []
        for _ in range(max(3, args.steps // 2)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            sa.forward(Q, K, V, rt, cfg_nr, out=On)
            e1.record()
            ts.append((e0, e1))
        torch.cuda.synchronize()
        nr_ms = median([a.elapsed_time(b) for a, b in ts])
        del On
        noresid = {"forward_ms_median": nr_ms, "forward_with_residual_ms_median": warm["forward_ms_median"],
                   "residual_share_of_forward": 1.0 - nr_ms / warm["forward_ms_median"],
                   "exact_tflops": exact_flops / (nr_ms * 1e-3) / 1e12,
                   "exact_frac_of_peak": exact_flops / (nr_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}

    dense_ms = None
    if not args.no_dense:
        Od = sa.dense_ref_gpu(Q, K, V, block_q=w.block_q)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record()
        for _ in range(reps):
            sa.dense_ref_gpu(Q, K, V, block_q=w.block_q, out=Od)
        e1.record()
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / reps

    traffic = load_traffic(w.name, args.tau_mode)
    out = {
        "metric": METRIC,
        "value": dense_flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32 in, bf16 products",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "block_q": w.block_q, "block_k": w.block_k, "tau": cfg.tau, "tau_mode": args.tau_mode, "proxy": args.proxy, "fused": args.fused,
                   "max_keep": cfg.max_keep, "n_dense_prefix": cfg.n_dense_prefix,
                   "kept_fraction": kept_frac},
        "roofline": {"bound": "mfma", "achieved": fwd_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": fwd_tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": "flash_kernel (sparse forward with residual)",
                     "flops_per_launch": exact_flops + resid_flops, "avg_launch_ms": fwd_ms},
        "route": {"ms": route_ms, "bytes": route_bytes, "bytes_read": route_read, "bytes_written": route_written,
                  "GB/s": route_gbs, "frac_hbm": route_gbs / PEAK_HBM_GBS,
                  "stream_copy_GB/s": stream_gbs, "frac_stream_copy": route_gbs / stream_gbs},
        "forward_ms": fwd_ms,
        "dense_ms": dense_ms,
        "speedup_vs_dense": (dense_ms / (route_ms + fwd_ms)) if dense_ms else None,
        "inverse_kept_fraction": 1.0 / kept_frac,
        # 1 / (kept + residual share of the dense flops): the speedup the algorithmic work allows
        "inverse_algorithmic_fraction": dense_flops / (exact_flops + resid_flops),
        "residual_flops_per_forward": resid_flops,
        "no_residual": noresid,
        "mfma_counters": load_mfma(w.name, args.tau_mode),
        "issued_mfma_flops_per_forward": issued,
        "issued_mfma_frac": issued / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "timing_warm": warm,
        "timing_cold": cold,
        "permute": permute_timing(sa, Q, w) if w.hilbert else None,
        "sparsepr": sparsepr_compare(sa, Q, K, V, rt, cfg, O, args.sparsepr) if args.sparsepr else None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, cfg, Qc, Kc, Vc)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    if args.with_copy:
        copy_calibration()


if __name__ == "__main__":
    main()
