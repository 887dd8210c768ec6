"""Turn two rocprofv3 counter runs of one ``bench.py --only`` leg into the HBM
traffic figure that bench.py reports as the roofline's ``traffic``.

Usage (on the GPU host, one counter per run, then here), for a target of
TARGETS (doc_attn_c5: the 1M-token layer's document partial pass, the bench
line's roofline kernel; doc_attn_c2: the 4B layer's):

    cd /tmp && export TMPDIR=/tmp
    timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d <F> -o f -- \\
        python3 <repo>/bench.py --only <leg> --steps <steps> --warmup 1 --cpu-seconds 0
    timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d <W> -o w -- \\
        python3 <repo>/bench.py --only <leg> --steps <steps> --warmup 1 --cpu-seconds 0
    python3 bench_traffic.py <target> <F> <W>

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch.  Both are scaled by
what they read for a copy of known size in the same runs: the leg clones a
CALIB_BYTES buffer four times with the runtime's copy kernel (the largest
copies of the run), so each of those reads and writes exactly that many bytes.
The result goes to profiles/traffic_<target>.json with the hash of the
attention sources it belongs to (bench.py reports it only while that hash
matches).
"""
import csv
import glob
import json
import os
import sys
from collections import defaultdict

import bench

TARGETS = {
    "doc_attn_c5": dict(kernel="attn_rows_lds", leg="c5_doc_partial", steps=8, algo=4 * 1048576 * 2 * 128 * 2,
                        what="split-K partial pass of the exact document attention (attn_rows_lds) over one "
                             "layer of the 1M-token stack (4 KV heads x 1,048,576 keys)"),
    "doc_attn_c2": dict(kernel="attn_rows_lds", leg="c2_doc_partial", steps=48, algo=8 * 61440 * 2 * 128 * 2,
                        what="split-K partial pass of the exact document attention (attn_rows_lds) on the "
                             "Qwen3-4B-shaped decode layer (8 KV heads x 61,440 keys)"),
}
COPY = "copyBuffer"


def per_dispatch(root, counter, kernel):
    """{'kernel': [KiB per dispatch of its most frequent launch shape], 'copy': [largest copies]}."""
    files = glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % root)
    sums = defaultdict(float)
    names, grids = {}, {}
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                key = (f, row.get("Dispatch_Id") or row.get("Correlation_Id"))
                sums[key] += float(row["Counter_Value"])
                names[key] = row.get("Kernel_Name", "")
                grids[key] = row.get("Grid_Size", "")
    shapes = defaultdict(int)
    for key in sums:
        if kernel in names[key]:
            shapes[grids[key]] += 1
    timed = max(shapes, key=shapes.get) if shapes else None
    out = {"kernel": [], "copy": []}
    for key, v in sums.items():
        if kernel in names[key] and grids[key] == timed:
            out["kernel"].append(v)
        elif COPY in names[key]:
            out["copy"].append(v)
    if out["copy"]:                      # the calibration copies: the largest cluster
        top = max(out["copy"])
        out["copy"] = [v for v in out["copy"] if v >= 0.8 * top]
    return out


def main():
    target, froot, wroot = sys.argv[1], sys.argv[2], sys.argv[3]
    t = TARGETS[target]
    f, w = per_dispatch(froot, "FETCH_SIZE", t["kernel"]), per_dispatch(wroot, "WRITE_SIZE", t["kernel"])
    if not f["kernel"] or not w["kernel"] or not f["copy"] or not w["copy"]:
        raise SystemExit("missing dispatches: %s" % {k: len(v) for k, v in list(f.items()) + list(w.items())})
    mean = lambda xs: sum(xs) / len(xs)
    fetch_scale = bench.CALIB_BYTES / (mean(f["copy"]) * 1024.0)
    write_scale = bench.CALIB_BYTES / (mean(w["copy"]) * 1024.0)
    fk, wk = mean(f["kernel"]), mean(w["kernel"])
    hbm = fk * 1024.0 * fetch_scale + wk * 1024.0 * write_scale
    cmd = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc %s --output-format csv -d <out> "
           "-o %s -- python3 <repo>/bench.py --only " + t["leg"] + " --steps %d --warmup 1 --cpu-seconds 0" % t["steps"])
    res = {
        "kernel": t["what"],
        "commands": [cmd % ("FETCH_SIZE", "f"), cmd % ("WRITE_SIZE", "w"),
                     "python3 bench_traffic.py %s <fetch out> <write out>" % target],
        "raw_kib_per_dispatch": {"fetch": fk, "write": wk, "dispatches": len(f["kernel"])},
        "calibration": {"copy_kernel": "the runtime's copy kernel cloning a %d-byte buffer, in the same runs"
                                       % bench.CALIB_BYTES,
                        "copies": len(f["copy"]), "fetch_scale": fetch_scale, "write_scale": write_scale},
        "hbm_bytes_per_launch": int(round(hbm)),
        "algorithmic_bytes_per_launch": t["algo"],
        "source_hash": bench.source_hash(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic_%s.json" % target)
    with open(path, "w") as fh:
        json.dump(res, fh, indent=1)
    print("| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) |")
    print("|---|---|---|---|")
    print("| %s | %d | %.1f | %.1f |" % (t["kernel"], len(f["kernel"]), fk, wk))
    print("fetch scale %.4f, write scale %.4f; %d B per launch = %.4f x algorithmic"
          % (fetch_scale, write_scale, hbm, hbm / t["algo"]))


if __name__ == "__main__":
    main()
