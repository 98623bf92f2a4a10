"""Summarise rocprofv3 CSV output of bench.py runs into short text tables.

    python -m gated_delta_rule_87_amd.rocprof_summary --workload prefill_T8192_H64 \\
        --trace DIR --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \\
        [--sq DIR ...] --command-file FILE --out-dir profiles

Inputs are the directories rocprofv3 wrote with --output-format csv:
  --trace        --kernel-trace --stats run (kernel_stats.csv)
  --fetch/write  --pmc FETCH_SIZE / --pmc WRITE_SIZE runs of the same bench command
  --copy-*       the same counters for `bench.py --copy-calibration` (a plain 1 GiB
                 device copy): each counter's reading for a known byte count gives
                 its scale factor (bytes per counted KiB)
  --sq           --pmc runs of SQ_* counters
Writes one <kernel>__<workload>.md per kernel of the profiled call, the
copy_calibration__1GiB.md table, and merges the per-launch HBM bytes into
traffic.json, keyed by workload and by the hash of the kernel sources (bench.py
reports a measured "traffic" only while that hash matches).
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNELS = ("kda_sched_kernel", "kda_intra_kernel", "kda_chain_kernel", "kda_scan_kernel", "kda_recurrent_kernel")
COPY_KERNEL = "__amd_rocclr_copyBuffer"
GIB = 1 << 30


def kernel_source_hash():
    """Same hash as bench.py: every file under the package's csrc/."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_87_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def short_name(kernel_name):
    for k in KERNELS:
        if k in kernel_name:
            return k
    return COPY_KERNEL if COPY_KERNEL in kernel_name else None


def one_file(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return files[0]


def counters(d):
    """{(kernel, counter): [value per dispatch]} from a --pmc run."""
    out = {}
    for r in csv.DictReader(open(one_file(d, "counter_collection.csv"))):
        k = short_name(r["Kernel_Name"])
        if k is None:
            continue
        out.setdefault((k, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    return out


def kernel_stats(d):
    """Per short kernel name; instantiations of one kernel (template arguments) are merged."""
    out = {}
    for r in csv.DictReader(open(one_file(d, "kernel_stats.csv"))):
        k = short_name(r["Name"])
        if k is None:
            continue
        e = out.setdefault(k, {"calls": 0, "total_ns": 0.0, "min_us": float("inf"), "max_us": 0.0})
        e["calls"] += int(r["Calls"])
        e["total_ns"] += float(r["TotalDurationNs"])
        e["min_us"] = min(e["min_us"], float(r["MinNs"]) / 1e3)
        e["max_us"] = max(e["max_us"], float(r["MaxNs"]) / 1e3)
    for e in out.values():
        e["avg_us"] = e["total_ns"] / e["calls"] / 1e3
    return out


def trace_durations(d):
    """{kernel: [duration us of each launch, in dispatch order]} from the kernel trace."""
    out = {}
    rows = list(csv.DictReader(open(one_file(d, "kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    for r in rows:
        k = short_name(r["Kernel_Name"])
        if k is not None:
            out.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--sq", action="append", default=[])
    ap.add_argument("--bench-json", help="bench.py output line of the same workload (algorithmic bytes)")
    ap.add_argument("--calls", type=int, default=0,
                    help="kda_fwd calls in the traced run (warm-up + timed), to pick out the timed launches")
    ap.add_argument("--command-file", required=True, help="text file holding the exact commands that were run")
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args()

    cf = counters(a.copy_fetch)[(COPY_KERNEL, "FETCH_SIZE")]
    cw = counters(a.copy_write)[(COPY_KERNEL, "WRITE_SIZE")]
    f_fetch = GIB / (statistics.mean(cf) * 1024)    # bytes really read per counted byte
    f_write = GIB / (statistics.mean(cw) * 1024)
    commands = open(a.command_file).read().strip()
    os.makedirs(a.out_dir, exist_ok=True)
    with open(os.path.join(a.out_dir, "copy_calibration__1GiB.md"), "w") as fh:
        fh.write("# HBM counter calibration: plain 1 GiB device-to-device copy\n\n")
        fh.write("Commands:\n\n```\n" + commands + "\n```\n\n")
        fh.write("| counter | mean KiB per copy launch | launches | bytes moved | scale factor |\n|---|---|---|---|---|\n")
        fh.write(f"| FETCH_SIZE | {statistics.mean(cf):.0f} | {len(cf)} | {GIB} read | {f_fetch:.4f} |\n")
        fh.write(f"| WRITE_SIZE | {statistics.mean(cw):.0f} | {len(cw)} | {GIB} written | {f_write:.4f} |\n\n")
        fh.write("Scaled bytes = counter KiB x 1024 x scale factor.\n")

    fetch, write = counters(a.fetch), counters(a.write)
    sq = {}
    for d in a.sq:
        sq.update(counters(d))
    stats = kernel_stats(a.trace)
    durations = trace_durations(a.trace)
    alg = {}
    if a.bench_json:
        line = open(a.bench_json).read().strip().splitlines()[-1]
        for k, v in json.loads(line).get("kernels", {}).items():
            alg[k] = v
    src_hash = kernel_source_hash()
    traffic = {}
    for k in KERNELS:
        if k not in stats:
            continue
        fk, wk = fetch.get((k, "FETCH_SIZE")), write.get((k, "WRITE_SIZE"))
        rd = statistics.mean(fk) * 1024 * f_fetch if fk else None
        wr = statistics.mean(wk) * 1024 * f_write if wk else None
        tot = (rd or 0) + (wr or 0) if (rd is not None and wr is not None) else None
        traffic[k] = {"hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
                      "hbm_bytes_per_launch": tot}
        st = stats[k]
        with open(os.path.join(a.out_dir, f"{k}__{a.workload}.md"), "w") as fh:
            fh.write(f"# {k} on workload {a.workload}\n\n")
            fh.write("Commands (run from /tmp with TMPDIR=/tmp; $R is the repository root):\n\n```\n" + commands + "\n```\n\n")
            fh.write(f"Kernel sources hash: `{src_hash}`\n\n")
            fh.write("## rocprofv3 --kernel-trace --stats\n\n| calls | average us | min us | max us |\n|---|---|---|---|\n")
            fh.write(f"| {st['calls']} | {st['avg_us']:.1f} | {st['min_us']:.1f} | {st['max_us']:.1f} |\n\n")
            if k in alg:
                # the timed calls are the last ones: average the trace over as many launches
                # (a segmented chain launches the chain kernel twice per call)
                per_call = max(1, round(st["calls"] / max(1, a.calls))) if a.calls else 1
                tail = durations.get(k, [])[-alg[k]["launches"] * per_call:]
                if tail and a.calls:
                    fh.write(f"The same trace over the last {len(tail)} launches (the timed calls, after the "
                             f"warm-up): {statistics.mean(tail):.1f} us average.\n\n")
                fh.write(f"bench.py (HIP events on the launch stream, same command without the profiler): "
                         f"{alg[k]['avg_ms'] * 1e3:.1f} us average over {alg[k]['launches']} calls")
                if per_call > 1:
                    fh.write(f", each interval the whole state-chain stage of a call ({per_call} launches of "
                             f"this kernel and the scan kernel between them)")
                fh.write(".\n\n")
            fh.write("## HBM traffic per launch (FETCH_SIZE, WRITE_SIZE; copy-calibrated)\n\n")
            fh.write("| counter | mean KiB per launch | scale | bytes |\n|---|---|---|---|\n")
            if fk:
                fh.write(f"| FETCH_SIZE | {statistics.mean(fk):.0f} | {f_fetch:.4f} | {rd:.4g} |\n")
            if wk:
                fh.write(f"| WRITE_SIZE | {statistics.mean(wk):.0f} | {f_write:.4f} | {wr:.4g} |\n")
            if tot is not None:
                fh.write(f"| total | | | {tot:.4g} |\n")
            if k in alg:
                fh.write(f"\nAlgorithmic bytes of this kernel: {alg[k]['alg_bytes']:.4g}")
                if alg[k]['design_bytes'] != alg[k]['alg_bytes']:
                    fh.write(f"; bytes the design moves (with the per-chunk records): {alg[k]['design_bytes']:.4g}")
                fh.write(".\n")
            rows = sorted((c, v) for (kk, c), v in sq.items() if kk == k)
            if rows:
                fh.write("\n## SQ counters (mean per launch)\n\n| counter | value |\n|---|---|\n")
                for c, v in rows:
                    fh.write(f"| {c} | {statistics.mean(v):.4g} |\n")
                waves = statistics.mean(sq[(k, "SQ_WAVES")]) if (k, "SQ_WAVES") in sq else None
                if waves:
                    fh.write("\nPer wave: " + ", ".join(
                        f"{c} {statistics.mean(sq[(k, c)]) / waves:.0f}" for c in
                        ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR")
                        if (k, c) in sq) + ".\n")

    path = os.path.join(a.out_dir, "traffic.json")
    try:
        doc = json.load(open(path))
    except (OSError, ValueError):
        doc = {}
    doc.setdefault("calibration", {})
    doc["calibration"] = {"fetch_scale": f_fetch, "write_scale": f_write,
                          "reference": "plain 1 GiB device-to-device copy (bench.py --copy-calibration)"}
    doc.setdefault("workloads", {})[a.workload] = {"source_hash": src_hash, "kernels": traffic}
    with open(path, "w") as fh:
        json.dump(doc, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({"workload": a.workload, "source_hash": src_hash, "traffic": traffic}, indent=1))


if __name__ == "__main__":
    main()
