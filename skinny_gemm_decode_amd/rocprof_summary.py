"""Summaries of rocprofv3 CSV output for this library's kernels.

    python -m skinny_gemm_decode_amd.rocprof_summary counters DIR [DIR ...]
        per-kernel mean / min / max of every counter in DIR/**/*counter_collection.csv
    python -m skinny_gemm_decode_amd.rocprof_summary stats DIR
        per-kernel calls and average / min / max duration from DIR/**/*kernel_stats.csv
    python -m skinny_gemm_decode_amd.rocprof_summary source-hash
        sha256 of the sources that define the bf16 M=1 GEMV kernel (a traffic
        figure measured with hardware counters is valid only for these sources)
    python -m skinny_gemm_decode_amd.rocprof_summary traffic-md FETCH_DIR WRITE_DIR
        markdown summary of the headline GEMV's HBM traffic from one FETCH_SIZE
        and one WRITE_SIZE pass of `bench.py --arms none --calibrate-copy`,
        scaled by what the counters read for a 256 MiB device copy
    python -m skinny_gemm_decode_amd.rocprof_summary trace-md DIR TITLE COMMAND
        markdown table of DIR/**/*kernel_stats.csv
    python -m skinny_gemm_decode_amd.rocprof_summary counters-md TITLE COMMAND DIR [DIR ...]
        markdown table of the per-dispatch mean of every counter, per kernel of
        this library, over the counter runs in the DIRs
"""

from __future__ import annotations

import collections
import csv
import glob
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))

#: sources that fully determine the GEMV kernels' code
GEMV_SOURCES = ["csrc/common.h", "csrc/gemv_impl.h", "csrc/gemv_instances.h", "csrc/gemv_bf16.hip"]


def gemv_source_hash() -> str:
    h = hashlib.sha256()
    for rel in GEMV_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def counters(dirs):
    out = []
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            acc = collections.defaultdict(list)
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    acc[(r["Kernel_Name"].split("(")[0], r["Counter_Name"])].append(float(r["Counter_Value"]))
            out.append(f"== {f}")
            for (k, c), v in sorted(acc.items(), key=lambda kv: -len(kv[1])):
                out.append(f"{c:12s} n={len(v):6d} mean={sum(v) / len(v):14.1f} min={min(v):14.1f} "
                           f"max={max(v):14.1f}  {k}")
    return "\n".join(out)


def stats(d):
    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        out.append(f"== {f}")
        with open(f) as fh:
            for r in csv.DictReader(fh):
                out.append(f"{r['Name'].split('(')[0]:80s} calls={r['Calls']:>7s} avg_us={float(r['AverageNs']) / 1e3:9.3f} "
                           f"min_us={float(r['MinNs']) / 1e3:9.3f} max_us={float(r['MaxNs']) / 1e3:9.3f}")
    return "\n".join(out)


def _counter_means(d, counter):
    """{kernel: (dispatches, mean, max)} of one counter over DIR/**/*counter_collection.csv."""
    acc = collections.defaultdict(list)
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    acc[r["Kernel_Name"].split("(")[0]].append(float(r["Counter_Value"]))
    return {k: (len(v), sum(v) / len(v), max(v)) for k, v in acc.items()}


COPY_BYTES = 1 << 28            # bench.py --calibrate-copy: 256 MiB device-to-device copies
HEADLINE_BYTES = 12288 * 4096 * 2 + 4096 * 2 + 12288 * 4   # weights + x + y of the headline GEMV


def traffic_md(fetch_dir, write_dir):
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    gemv = max((k for k in fetch if k.startswith("void skg::gemv_kernel<0, 1,")), key=lambda k: fetch[k][0])
    read = next(k for k in fetch if "stream_read_kernel" in k)
    copy = next(k for k in fetch if "copyBuffer" in k)
    # the copy's largest dispatch is the 256 MiB one (read and write COPY_BYTES)
    f_copy, w_copy = fetch[copy][2], write[copy][2]
    f_scale = COPY_BYTES / 1024.0 / f_copy
    w_scale = COPY_BYTES / 1024.0 / w_copy
    fg, wg = fetch[gemv][1], write.get(gemv, (0, 0.0, 0.0))[1]
    traffic = int(round((fg * f_scale + wg * w_scale) * 1024))
    lines = [
        "# HBM traffic of the bf16 GEMV M=1 K=4096 N=12288 (hardware counters)",
        "",
        "Two counter runs of the same command, one counter each (run from the repository root on one MI355X):",
        "",
        f"    rocprofv3 --pmc FETCH_SIZE -f csv -d {fetch_dir} -o run -- python -u bench.py --arms none "
        "--no-cpu-baseline --steps 10 --warmup 0 --calibrate-copy",
        f"    rocprofv3 --pmc WRITE_SIZE -f csv -d {write_dir} -o run -- python -u bench.py --arms none "
        "--no-cpu-baseline --steps 10 --warmup 0 --calibrate-copy",
        f"    python -m skinny_gemm_decode_amd.rocprof_summary traffic-md {fetch_dir} {write_dir}",
        "",
        "Per-dispatch means (KiB):",
        "",
        "| kernel | dispatches | FETCH_SIZE | WRITE_SIZE |",
        "|---|---|---|---|",
        f"| `{gemv}` (bf16 M=1 default) | {fetch[gemv][0]} | {fg:.1f} | {wg:.1f} |",
        f"| `{read}` over the same 100,663,296-byte buffers | {fetch[read][0]} | {fetch[read][1]:.1f} | "
        f"{write.get(read, (0, 0.0, 0.0))[1]:.1f} |",
        f"| `{copy}`, 256 MiB device-to-device copy (largest dispatch) | {fetch[copy][0]} | {f_copy:.1f} | {w_copy:.1f} |",
        "",
        f"Calibration against the plain copy of known size ({COPY_BYTES:,} bytes read and written): FETCH_SIZE is "
        f"scaled by {f_scale:.4f} and WRITE_SIZE by {w_scale:.4f} (counter KiB to bytes read / written).",
        "",
        f"Scaled traffic per GEMV launch: {fg:.1f} x {f_scale:.4f} + {wg:.1f} x {w_scale:.4f} KiB = {traffic:,} bytes, "
        f"against {HEADLINE_BYTES:,} algorithmic bytes (weights 100,663,296 + x 8,192 + y 49,152): "
        f"{traffic / HEADLINE_BYTES:.4f}x.",
        "",
        "Machine-readable (bench.py reports this traffic only while the GEMV sources hash to this value):",
        "",
        f"    traffic_bytes_per_launch: {traffic}",
        f"    gemv_source_sha256: {gemv_source_hash()}",
    ]
    return "\n".join(lines)


def trace_md(d, title, command):
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Name"].split("(")[0]
                if "skg::" not in name:
                    continue
                rows.append((name, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                             float(r["MaxNs"]) / 1e3))
    lines = [f"# Kernel-trace summary: {title}", "", "Command (run from the repository root on one MI355X):", "",
             f"    {command}", "", "Source: `run_kernel_stats.csv` (this library's kernels only).", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for name, calls, avg, mn, mx in sorted(rows, key=lambda r: -r[1] * r[2]):
        lines.append(f"| `{name}` | {calls} | {avg:.3f} | {mn:.3f} | {mx:.3f} |")
    return "\n".join(lines)


def counters_md(title, command, dirs):
    means = collections.defaultdict(dict)
    calls = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            acc = collections.defaultdict(list)
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    k = r["Kernel_Name"].split("(")[0]
                    if "skg::" in k:
                        acc[(k, r["Counter_Name"])].append(float(r["Counter_Value"]))
            for (k, c), v in acc.items():
                means[k][c] = sum(v) / len(v)
                calls[k] = max(calls.get(k, 0), len(v))
    names = sorted({c for m in means.values() for c in m})
    lines = [f"# Hardware counters: {title}", "", "Commands (run from the repository root on one MI355X, one counter",
             "set per run):", ""] + [f"    {c}" for c in command.split(" ;; ")] + [
             "", "Per-dispatch means over every dispatch of each kernel:", "",
             "| kernel | dispatches | " + " | ".join(names) + " |", "|---|---|" + "---|" * len(names)]
    for k in sorted(means, key=lambda k: -calls[k]):
        lines.append(f"| `{k}` | {calls[k]} | " + " | ".join(
            f"{means[k][c]:.4g}" if c in means[k] else "" for c in names) + " |")
    return "\n".join(lines)


def main(argv):
    if len(argv) >= 2 and argv[0] == "counters":
        print(counters(argv[1:]))
    elif len(argv) == 2 and argv[0] == "stats":
        print(stats(argv[1]))
    elif argv == ["source-hash"]:
        print(gemv_source_hash())
    elif len(argv) == 3 and argv[0] == "traffic-md":
        print(traffic_md(argv[1], argv[2]))
    elif len(argv) == 4 and argv[0] == "trace-md":
        print(trace_md(argv[1], argv[2], argv[3]))
    elif len(argv) >= 4 and argv[0] == "counters-md":
        print(counters_md(argv[1], argv[2], argv[3:]))
    else:
        print(__doc__, file=sys.stderr)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
