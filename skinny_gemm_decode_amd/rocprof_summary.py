"""Summaries of rocprofv3 CSV output for this library's kernels.

    python -m skinny_gemm_decode_amd.rocprof_summary counters DIR [DIR ...]
        per-kernel mean / min / max of every counter in DIR/**/*counter_collection.csv
    python -m skinny_gemm_decode_amd.rocprof_summary stats DIR
        per-kernel calls and average / min / max duration from DIR/**/*kernel_stats.csv
    python -m skinny_gemm_decode_amd.rocprof_summary source-hash
        sha256 of the sources that define the bf16 M=1 GEMV kernel (a traffic
        figure measured with hardware counters is valid only for these sources)
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


def main(argv):
    if len(argv) >= 2 and argv[0] == "counters":
        print(counters(argv[1:]))
    elif len(argv) == 2 and argv[0] == "stats":
        print(stats(argv[1]))
    elif argv == ["source-hash"]:
        print(gemv_source_hash())
    else:
        print(__doc__, file=sys.stderr)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
