"""Short text summaries of rocprofv3 output for the profiles/ folder.

rocprofv3 writes one CSV row per dispatch (kernel trace) or per dispatch and counter
(counter collection). These summaries keep what the measurements use: per kernel and
grid size the dispatch count and the mean, min and max duration, or the mean of each
counter; every summary is stamped with the digest of the kernel sources it was taken on
(the same digest bench.py checks before it uses a counted figure).

Usage (on the machine that ran the profiler):
  python -m kv_cache_bit_amd.profsum trace    <..._kernel_trace.csv>       [--match NAME]
  python -m kv_cache_bit_amd.profsum counters <..._counter_collection.csv> [--match NAME]
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ["kv_cache_bit_amd/csrc/kvarn_common.h", "kv_cache_bit_amd/csrc/kvarn_launch.h",
           "kv_cache_bit_amd/csrc/quantize.hip", "kv_cache_bit_amd/csrc/quantize_dev.h",
           "kv_cache_bit_amd/csrc/attn.hip", "kv_cache_bit_amd/csrc/dequant.hip"]


def source_digest(files=SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    n = name
    for p in ("void ", "(anonymous namespace)::", "kvarn::"):
        if n.startswith(p):
            n = n[len(p):]
    return n.split("(")[0].strip()


def _grid(r) -> int:
    for k in ("Grid_Size", "Grid_Size_X", "Grid_X"):
        if k in r and r[k] not in ("", None):
            try:
                return int(float(r[k]))
            except ValueError:
                pass
    return -1


def trace(path: str, match: str | None) -> list[str]:
    csv.field_size_limit(1 << 30)
    durs = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            name = short_name(r.get("Kernel_Name", ""))
            if match and match not in name:
                continue
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            durs[(name, _grid(r))].append((t1 - t0) / 1e3)
    total = sum(sum(v) for v in durs.values()) or 1.0
    out = [f"{'kernel':48s} {'grid':>10s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share':>6s}"]
    for (name, grid), v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{name[:48]:48s} {grid:10d} {len(v):6d} {statistics.mean(v):9.2f} {min(v):9.2f} "
                   f"{max(v):9.2f} {100 * sum(v) / total:5.1f}%")
    return out


def counters(path: str, match: str | None) -> list[str]:
    csv.field_size_limit(1 << 30)
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(path) as f:
        for r in csv.DictReader(f):
            name = short_name(r.get("Kernel_Name", ""))
            if match and match not in name:
                continue
            vals[(name, _grid(r))][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = []
    for key in sorted(vals):
        out.append(f"[{key[0]}] grid {key[1]}")
        for c in sorted(vals[key]):
            v = vals[key][c]
            out.append(f"  {c} = {statistics.mean(v):.1f}   (dispatches {len(v)})")
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("mode", choices=("trace", "counters"))
    ap.add_argument("csv")
    ap.add_argument("--match", default=None, help="keep kernels whose short name contains this")
    a = ap.parse_args(argv)
    lines = trace(a.csv, a.match) if a.mode == "trace" else counters(a.csv, a.match)
    print("\n".join(lines))
    print(f"source_digest = {source_digest()}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
