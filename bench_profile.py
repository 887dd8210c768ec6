"""Summarise a rocprofv3 kernel trace (``<out>/<name>_kernel_trace.csv``) as the
tables kept under profiles/: per kernel launch shape (kernel, blocks) the
number of launches and the average, median, minimum and maximum duration in
microseconds, first launch first; with ``--kernel K --last N`` also the
average of the last N launches of kernel K (the timed window of a bench leg
whose earlier launches are its warm-up).

    python3 bench_profile.py <trace.csv> [--kernel attn_rows_lds --last 56]
"""
import argparse
import csv
from collections import OrderedDict


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("trace")
    ap.add_argument("--kernel", default=None)
    ap.add_argument("--last", type=int, default=0)
    ap.add_argument("--skip", default="at::native", help="kernels whose name contains this are left out")
    args = ap.parse_args()
    rows = list(csv.DictReader(open(args.trace)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    agg = OrderedDict()
    named = []
    for r in rows:
        name = r["Kernel_Name"].split("(")[0].replace("void ", "").strip()
        if args.skip and args.skip in name:
            continue
        wg = int(r.get("Workgroup_Size_X") or r.get("Workgroup_Size") or 1)
        grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        agg.setdefault((name[:64], grid // max(wg, 1)), []).append(us)
        if args.kernel and args.kernel in name:
            named.append(us)
    print("| kernel | blocks | launches | avg us | median us | min us | max us |")
    print("|---|---|---|---|---|---|---|")
    for (name, blocks), ds in agg.items():
        s = sorted(ds)
        print("| `%s` | %d | %d | %.2f | %.2f | %.2f | %.2f |"
              % (name, blocks, len(ds), sum(ds) / len(ds), s[len(s) // 2], s[0], s[-1]))
    if args.kernel and args.last:
        tail = named[-args.last:]
        print("\nlast %d launches of %s: average %.2f us (min %.2f, max %.2f)"
              % (len(tail), args.kernel, sum(tail) / len(tail), min(tail), max(tail)))


if __name__ == "__main__":
    main()
