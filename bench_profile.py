"""Summarise a rocprofv3 kernel trace (``<out>/<name>_kernel_trace.csv``) as the
tables kept under profiles/: per kernel launch shape (kernel, blocks) the
number of launches and the average, median, minimum and maximum duration in
microseconds, first launch first; with ``--kernel K --last N`` also the
average of the last N launches of kernel K (the timed window of a bench leg
whose earlier launches are its warm-up).

    python3 bench_profile.py <trace.csv> [--kernel attn_rows_lds --last 56]

With ``--counters`` the file is a counter_collection.csv (``rocprofv3 --pmc``):
per dispatch of kernel K (its most frequent launch shape) every counter is
summed over its instances, and the table gives the average per dispatch; MFMA
busy per SIMD = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1,024 SIMDs), the
GRBM counter being summed over the 8 XCDs.

    python3 bench_profile.py <counter_collection.csv> --counters --kernel attn_rows_lds32
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
    ap.add_argument("--counters", action="store_true")
    args = ap.parse_args()
    if args.counters:
        return counters(args)
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


def counters(args):
    from collections import defaultdict
    per = defaultdict(lambda: defaultdict(float))     # dispatch -> counter -> sum over instances
    grid = {}
    for r in csv.DictReader(open(args.trace)):
        if args.kernel not in r.get("Kernel_Name", ""):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        grid[key] = r.get("Grid_Size", "")
    shapes = defaultdict(int)
    for k in per:
        shapes[grid[k]] += 1
    timed = max(shapes, key=shapes.get)
    keys = [k for k in per if grid[k] == timed]
    names = sorted({c for k in keys for c in per[k]})
    print("%d dispatches of %s (grid %s)\n" % (len(keys), args.kernel, timed))
    print("| counter | average per dispatch |")
    print("|---|---|")
    avg = {c: sum(per[k][c] for k in keys) / len(keys) for c in names}
    for c in names:
        print("| %s | %.6g |" % (c, avg[c]))
    if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg:
        # GRBM_GUI_ACTIVE comes summed over the 8 XCDs' instances: / 8 = the kernel's cycles
        cyc = avg["GRBM_GUI_ACTIVE"] / 8
        print("\nkernel cycles %.4g; MFMA busy per SIMD: %.3f" % (cyc, avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 1024)))
        if "SQ_INSTS_VALU" in avg:
            print("VALU issue per SIMD (4 cycles a wave64 instruction): %.3f; VALU instructions per MFMA: %.1f"
                  % (4 * avg["SQ_INSTS_VALU"] / (cyc * 1024), avg["SQ_INSTS_VALU"] / max(avg.get("SQ_INSTS_MFMA", 0), 1)))


if __name__ == "__main__":
    main()
