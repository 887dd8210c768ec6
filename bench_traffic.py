"""Turn two rocprofv3 counter runs of ``bench.py --only doc_partial`` into the
HBM traffic figure that bench.py reports as ``roofline.traffic``.

Usage (on the GPU host, one counter per run, then here):

    cd /tmp && export TMPDIR=/tmp
    timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d <F> -o f -- \
        python3 <repo>/bench.py --only doc_partial --steps 24 --warmup 24 --cpu-seconds 0
    timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d <W> -o w -- \
        python3 <repo>/bench.py --only doc_partial --steps 24 --warmup 24 --cpu-seconds 0
    python3 bench_traffic.py <F> <W>

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch.  Both are scaled by
what they read for a copy of known size in the same runs: bench.py clones the
125,829,120-byte document K and V caches of the Qwen3-4B-shaped layer into its
layer replicas with the runtime's copy kernel (one dispatch per clone, the
largest copies of the run), so each of those reads and writes exactly that
many bytes.  The result is written to
profiles/traffic_doc_attn_c2.json together with the hash of the attention
sources it belongs to (bench.py reports it only while that hash matches).
"""
import csv
import glob
import json
import os
import sys
from collections import defaultdict

import bench

COPY_BYTES = 8 * 61440 * 128 * 2          # one of K, V of the 4B layer
ALGO_BYTES = 2 * COPY_BYTES               # K and V read once per launch
KERNEL = "attn_partial_mfma"
COPY = "copyBuffer"


def per_dispatch(root, counter):
    """{kernel substring: [KiB per dispatch]} for the partial pass and the copies."""
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
    out = {KERNEL: [], COPY: []}
    # the timed launch shape: the partial pass also runs once or twice in other
    # shapes while the script warms the other entry points
    shapes = defaultdict(int)
    for key in sums:
        if KERNEL in names[key]:
            shapes[grids[key]] += 1
    timed = max(shapes, key=shapes.get) if shapes else None
    for key, v in sums.items():
        if KERNEL in names[key] and grids[key] == timed:
            out[KERNEL].append(v)
        elif COPY in names[key]:
            out[COPY].append(v)
    # the copies also clone the module weights and the local caches (10 to 100
    # times smaller): keep the K and V clones, the largest cluster
    if out[COPY]:
        top = max(out[COPY])
        out[COPY] = [v for v in out[COPY] if v >= 0.5 * top]
    return out


def main():
    froot, wroot = sys.argv[1], sys.argv[2]
    f, w = per_dispatch(froot, "FETCH_SIZE"), per_dispatch(wroot, "WRITE_SIZE")
    if not f[KERNEL] or not w[KERNEL] or not f[COPY] or not w[COPY]:
        raise SystemExit("missing dispatches: %s" % {k: len(v) for k, v in list(f.items()) + list(w.items())})
    mean = lambda xs: sum(xs) / len(xs)
    fetch_scale = COPY_BYTES / (mean(f[COPY]) * 1024.0)
    write_scale = COPY_BYTES / (mean(w[COPY]) * 1024.0)
    fk, wk = mean(f[KERNEL]), mean(w[KERNEL])
    hbm = fk * 1024.0 * fetch_scale + wk * 1024.0 * write_scale
    cmd = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc %s --output-format csv -d <out> "
           "-o %s -- python3 <repo>/bench.py --only doc_partial --steps 24 --warmup 24 --cpu-seconds 0")
    res = {
        "kernel": "split-K partial pass of the exact document attention (attn_partial_mfma) on the "
                  "Qwen3-4B-shaped decode layer",
        "commands": [cmd % ("FETCH_SIZE", "f"), cmd % ("WRITE_SIZE", "w"),
                     "python3 bench_traffic.py <fetch out> <write out>"],
        "raw_kib_per_dispatch": {"fetch": fk, "write": wk, "dispatches": len(f[KERNEL])},
        "calibration": {"copy_kernel": "the runtime's copy kernel cloning the %d-byte document K and V caches "
                                       "into the layer replicas, in the same runs" % COPY_BYTES,
                        "copies": len(f[COPY]), "fetch_scale": fetch_scale, "write_scale": write_scale},
        "hbm_bytes_per_launch": int(round(hbm)),
        "algorithmic_bytes_per_launch": ALGO_BYTES,
        "source_hash": bench.source_hash(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic_doc_attn_c2.json")
    with open(path, "w") as fh:
        json.dump(res, fh, indent=1)
    print("| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) |")
    print("|---|---|---|---|")
    print("| attn_partial_mfma | %d | %.1f | %.1f |" % (len(f[KERNEL]), fk, wk))
    print("fetch scale %.4f, write scale %.4f; %d B per launch = %.4f x algorithmic"
          % (fetch_scale, write_scale, hbm, hbm / ALGO_BYTES))


if __name__ == "__main__":
    main()
