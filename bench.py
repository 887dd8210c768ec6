#!/usr/bin/env python3
"""Benchmark of the Nectar attention hot path on one MI355X.

Headline workload: the Qwen2.5-7B-1M-shaped 28-layer stack with a 1M-token
document (4 KV heads, 28 query heads, d = 128, bf16; n = 1,048,576 document
keys per layer and KV head, 60 GB of document cache resident in HBM; 8
questions decoding one token each, 256 prompt tokens then 128 decode steps).
A step is one decode step of the whole stack, every layer in turn, through the
three forms of the document part:

  Nectar (the headline `value`): per layer the MLP module forward (target
      128->5120->128, score 128->3072->1, GELU) and causal local attention over
      the question's own tokens, merged by log-sum-exp (Eqs. (3.4)-(3.5));
  Quadrature: the same with the learnable-KV-pair module (p = 10,486 pairs);
  exact: exact attention over all 1,048,576 document keys, merged likewise.

Each path of each decode step is one HIP graph of its 28 layer steps (the
layers' caches, modules and queries are their own), replayed on the current
stream; HIP events between the paths of every step give the per-step times.
`--warmup` steps run untimed, then exactly `--steps` steps are timed; decode
step s of the stack sees 257 + s local keys (s = step index modulo 128).
`value` = query tokens per second per layer of the Nectar path (8 tokens x 28
layers per step over the Nectar share of the step time); `paths` gives all
three; `timing` the per-step median and 10th/90th percentiles and the device
clocks read while steps run.  Inputs are resident in HBM before timing (the
boundary takes device buffers, so there is no host-transfer rate to report).
The stack's tensors are N(0, 1) draws from a seeded device generator (modules
N(0, 1/fan_in)): a rotation leaves an N(0, 1) key N(0, 1), so RoPE'd keys and
these draws have the same distribution.

`roofline` covers the exact path's dominant kernel, the split-K partial pass
of the document attention over a layer's 1,048,576 keys (one launch per layer:
Hkv x n x 2 x d x 2 = 2,147,483,648 algorithmic bytes), timed alone over the
28 layers' caches with HIP events; `traffic` comes from the counter summary in
profiles/ while the kernel's sources are unchanged.  `cpu_baseline` times the
fp64 CPU oracle on the host cores: the Nectar path on one decode step of one
layer, and slices of every workload and form (exact, MLP, Quadrature, local
attention, merge).  `pages_context` quotes the only timing figures the pages
give (end-to-end generation, hardware not stated).  Extras: the
Qwen3-4B-shaped decode layer (fused step, each path, components, its own
document-pass roofline), per-layer timings of the batch-64 decode and prefill
workloads, the batched-prefill MLP against the MFMA peak, and the NEXT kernels.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# sources of the document-attention partial pass (the traffic figures are valid
# while these hash to the value stored with them)
ATTN_SOURCES = ["learned_kv_cache_02_amd/csrc/" + f for f in
                ("attn.hip", "attn_body.hpp", "attn_common.hpp", "attn_lds.hip", "lds_common.hpp",
                 "device_common.hpp", "kernels.hpp")]
CALIB_BYTES = 1 << 30   # runtime copies of this many bytes (the largest of a profiling run) calibrate the counters

# The pages' own timing figures (Nectar notes, section 4.8, App. D, Table 12):
# end-to-end generation, base model with the full document in context versus
# Nectar; the hardware is not stated.  Context only.
PAGES_TABLE12 = {
    "source": "Nectar notes, section 4.8 / App. D, Table 12 (end-to-end generation; hardware not stated)",
    "rows": [
        {"model": "Qwen3-1.7B", "doc_tokens": 40022, "ttft_base": "183,000 (unit garbled; ms)",
         "ttft_nectar_ms": 26.4, "decode_tok_s": [9.5, 44.2], "peak_mem_gb": [24.9, 7.7]},
        {"model": "Qwen3-1.7B", "doc_tokens": 122466, "ttft_base": "299,900 (unit garbled; ms)",
         "ttft_nectar_ms": 29.3, "decode_tok_s": [4.4, 37.7], "peak_mem_gb": [60.4, 8.2]},
        {"model": "Qwen3-4B", "doc_tokens": 40022, "ttft_base": "347,900 (unit garbled; ms)",
         "ttft_nectar_ms": 44.6, "decode_tok_s": [6.3, 18.4], "peak_mem_gb": [38.6, 16.7]},
        {"model": "Qwen3-4B", "doc_tokens": 122466, "ttft_base": "557,600 (unit garbled; ms)",
         "ttft_nectar_ms": 50.1, "decode_tok_s": [1.5, 15.7], "peak_mem_gb": [84.2, 17.1]},
    ],
    "hardware": "not stated",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="CPU oracle budget of the headline sample (0: skip every CPU leg)")
    ap.add_argument("--only", default=None,
                    choices=["stack", "c5_doc_partial", "c4_doc_partial", "c3_mlp10", "c2_doc_partial", "train_step",
                             "deep_modules"],
                    help="time one leg only (profiling runs): the stack, one kernel's launches, the "
                         "module's training step, or the deep modules")
    ap.add_argument("--no-extras", action="store_true", help="skip the extra workloads and kernels")
    return ap.parse_args()


def source_hash():
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(name):
    """HBM bytes per launch of a profiled kernel, if its sources are unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        tj = json.load(fh)
    return tj.get("hbm_bytes_per_launch") if tj.get("source_hash") == source_hash() else None


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from learned_kv_cache_02_amd import configs, nectar, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only in ("c4_doc_partial", "c3_mlp10", "c2_doc_partial"):
        print(json.dumps(profile_leg(torch, np, nectar, configs, synth, dev, args)), flush=True)
        return
    if args.only == "train_step":
        print(json.dumps(train_step_bench(torch, nectar, configs, dev)), flush=True)
        return
    if args.only == "deep_modules":
        print(json.dumps(deep_modules(torch, nectar, configs, dev)), flush=True)
        return

    res = {
        "metric": "query-tokens/s/layer, Nectar vs exact cache attn; % of HBM / MFMA roofline",
        "unit": "query-tokens/s/layer",
        "higher_is_better": True,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    st = stack_c5(torch, nectar, configs, dev, args)
    res.update(st.pop("line"))
    res.update(st)
    if args.only:
        print(json.dumps(res), flush=True)
        return
    torch.cuda.empty_cache()
    if not args.no_extras:
        res["c2_layer"] = c2_layer(torch, np, nectar, configs, synth, dev)
        torch.cuda.empty_cache()
        res["prefill_mlp"] = prefill_mlp(torch, np, nectar, configs, synth, dev)
        res["merge_k"] = merge_k_prefill(torch, nectar, configs, dev)
        res["fit_metrics"] = fit_metrics_prefill(torch, nectar, configs, dev)
        res["deep_modules"] = deep_modules(torch, nectar, configs, dev)
        res["train_step"] = train_step_bench(torch, nectar, configs, dev)
        res["workloads"] = {c.name: workload_layer(torch, nectar, c, dev) for c in (configs.C4, configs.C3)}
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(np, configs, synth, args.cpu_seconds)
    res["pages_context"] = PAGES_TABLE12
    print(json.dumps(res), flush=True)


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _pct(xs, f):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(round(f * (len(xs) - 1))))]


def stack_c5(torch, nectar, configs, dev, args):
    """The 28-layer 1M-token decode stack: every layer's document cache (60 GB),
    MLP and Quadrature modules, local caches and per-step queries on the device;
    per-step graphs of the three paths; the timed steps; the roofline kernel."""
    cfg = configs.C5
    L, Hkv, Hq, d, n, B, R = cfg.layers, cfg.Hkv, cfg.Hq, cfg.d, cfg.n, cfg.B, cfg.R
    m = cfg.mlps[0]
    bf = torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(2000 + cfg.seed)
    only = args.only

    def rn(*shape, std=1.0):
        # N(0, std^2) in bf16, drawn in chunks of 2^27 elements (bounded fp32 scratch)
        out = torch.empty(shape, dtype=bf, device=dev)
        flat = out.view(-1)
        for lo in range(0, flat.numel(), 1 << 27):
            hi = min(flat.numel(), lo + (1 << 27))
            flat[lo:hi] = (torch.randn(hi - lo, generator=g, device=dev) * std).to(bf)
        return out

    t0 = time.time()
    # each layer's document cache: one [Hkv][n][2][d] array, K and V interleaved by
    # key (a KV head's key range streams as one contiguous range)
    KV = [rn(Hkv, n, 2, d) for _ in range(L)]
    K = [x[:, :, 0] for x in KV]
    V = [x[:, :, 1] for x in KV]
    steps_total = args.warmup + args.steps
    z = lambda *s: torch.zeros(*s, device=dev)
    layers = []
    if only != "c5_doc_partial":
        for l in range(L):
            layers.append(dict(
                q=[rn(R, Hq, d) for _ in range(steps_total)],
                Kl=rn(B, Hkv, cfg.T_cap, d), Vl=rn(B, Hkv, cfg.T_cap, d),
                mlp=nectar.MLPModule(rn(Hkv, m.Ht, d, std=d ** -0.5), z(Hkv, m.Ht), rn(Hkv, m.Ht, d, std=m.Ht ** -0.5),
                                     z(Hkv, d), rn(Hkv, m.Hs, d, std=d ** -0.5), z(Hkv, m.Hs),
                                     rn(Hkv, m.Hs, std=m.Hs ** -0.5), z(Hkv)),
                kvp=nectar.KVPairModule(rn(Hkv, cfg.kv_pairs, d), rn(Hkv, cfg.kv_pairs, d))))
    torch.cuda.synchronize()
    print("stack: %d layers generated in %.1f s" % (L, time.time() - t0), file=sys.stderr, flush=True)
    doc_bytes = Hkv * n * 2 * d * 2
    line = {}
    extra = {}

    # --- the roofline kernel: the document partial pass of every layer (one launch each)
    dsc = nectar.desc(R, Hq, Hkv, d, nectar.BF16)
    part = torch.empty(max(16, nectar.doc_attn_partials_size(dsc, n)), dtype=torch.uint8, device=dev)
    q0 = rn(R, Hq, d)

    def doc_partials():
        for l in range(L):
            nectar.doc_attn_partials(q0, K[l], V[l], Hkv, partials=part)
    if only == "c5_doc_partial":
        # runtime copies of a known size in the same run calibrate the traffic counters
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        for _ in range(4):
            src.clone()
    doc_partials()
    torch.cuda.synchronize()
    gdoc = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gdoc):
        doc_partials()
    reps = max(1, args.steps // 4) if only == "c5_doc_partial" else 3
    gdoc.replay()
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 2)
    e0.record()
    for _ in range(reps):
        gdoc.replay()
    e1.record()
    torch.cuda.synchronize()
    us_doc = e0.elapsed_time(e1) / (reps * L) * 1e3
    ach = doc_bytes / (us_doc * 1e-6) / 1e9
    extra["roofline"] = {
        "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
        "traffic": load_traffic("doc_attn_c5"),
        "kernel": "split-K partial pass of the exact document attention over one layer's 1,048,576 keys "
                  "(nectar_doc_attn_partials: attn_rows_lds, one launch per layer), %.2f us per launch "
                  "(%d launches over the 28 layers' caches), %d algorithmic bytes per launch"
                  % (us_doc, reps * L, doc_bytes)}
    del gdoc
    if only == "c5_doc_partial":
        line["config"] = {"workload": "c5_qwen25_7b_1m_decode: document partial pass alone, 28 layer caches"}
        return dict(extra, line=line)

    # --- per-step graphs of the three paths through the stack
    f32 = dict(dtype=torch.float32, device=dev)
    outs = {"nectar": {"out_nectar": torch.empty(R, Hq, d, dtype=bf, device=dev), "lse_nectar": torch.empty(R, Hq, **f32)},
            "kvpair": {"out_nectar": torch.empty(R, Hq, d, dtype=bf, device=dev), "lse_nectar": torch.empty(R, Hq, **f32)},
            "exact": {"out_exact": torch.empty(R, Hq, d, dtype=bf, device=dev), "lse_exact": torch.empty(R, Hq, **f32)}}

    def path(name, s):
        ds = s % cfg.decode_steps
        kw = dict(B=B, Tq=1, T_loc=cfg.local_len(ds), q_offset=cfg.q_offset(ds), out=outs[name])
        for l, ly in enumerate(layers):
            if name == "exact":
                nectar.layer_step(ly["q"][s], ly["Kl"], ly["Vl"], Hkv, k=K[l], v=V[l], module=None, exact=True, **kw)
            else:
                nectar.layer_step(ly["q"][s], ly["Kl"], ly["Vl"], Hkv, module=ly["mlp" if name == "nectar" else "kvp"],
                                  exact=False, **kw)

    names = ["nectar", "kvpair", "exact"]
    for nm in names:                 # eager once: the binding's workspace outside any capture
        path(nm, steps_total - 1)
    torch.cuda.synchronize()
    graphs = {nm: [] for nm in names}
    for s in range(steps_total):
        for nm in names:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                path(nm, s)
            graphs[nm].append(gr)
    torch.cuda.synchronize()
    # Each path decodes its own consecutive steps -- its warm-up steps, then the
    # timed ones -- as a deployment of that path runs: a Nectar step then follows
    # a Nectar step, not a 60 GB exact step that leaves its TLB and caches cold.
    per = {nm: [] for nm in names}
    total_ms = 0.0
    for nm in names:
        for s in range(args.warmup):
            graphs[nm][s].replay()
        ev = _events(torch, 1 + args.steps)
        ev[0].record()
        for i in range(args.steps):
            graphs[nm][args.warmup + i].replay()
            ev[1 + i].record()
        torch.cuda.synchronize()
        per[nm] = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]     # ms
        total_ms += ev[0].elapsed_time(ev[args.steps])
    # the same timed steps with the three paths interleaved step by step (context)
    ev = _events(torch, 1 + 3 * args.steps)
    ev[0].record()
    for i in range(args.steps):
        for j, nm in enumerate(names):
            graphs[nm][args.warmup + i].replay()
            ev[1 + 3 * i + j].record()
    torch.cuda.synchronize()
    inter = {nm: [ev[3 * i + j].elapsed_time(ev[1 + 3 * i + j]) for i in range(args.steps)]
             for j, nm in enumerate(names)}
    # the clocks while steps run: about a second of Nectar steps enqueued, then read
    for _ in range(max(1, int(1.0 / max(1e-6, sum(per["nectar"]) / len(per["nectar"]) * 1e-3)))):
        graphs["nectar"][args.warmup].replay()
    clocks = gpu_clocks()
    torch.cuda.synchronize()
    for nm in ("out_nectar", "out_exact"):
        for o in outs.values():
            if nm in o and not torch.isfinite(o[nm].float()).all():
                raise RuntimeError("non-finite output in %s" % nm)
    tokens = R * L                    # query tokens per step through the stack
    mean = lambda xs: sum(xs) / len(xs)
    paths = {}
    for nm in names:
        ms = mean(per[nm])
        paths[nm] = {"qtok_s_layer": tokens / (ms * 1e-3), "ms_per_step": ms, "us_per_layer": ms * 1e3 / L,
                     "ms_per_step_median": _pct(per[nm], 0.5), "p10": _pct(per[nm], 0.1), "p90": _pct(per[nm], 0.9)}
    paths["nectar"]["form"] = "MLP 5120/3072 GELU (rho = %.4f)" % cfg.rho(m.params(d))
    paths["kvpair"]["form"] = "Quadrature, p = %d pairs (rho = %.4f)" % (cfg.kv_pairs, cfg.rho(2 * cfg.kv_pairs * d))
    paths["exact"]["form"] = "exact attention over 1,048,576 document keys"
    paths["nectar_speedup_vs_exact"] = paths["exact"]["ms_per_step"] / paths["nectar"]["ms_per_step"]
    paths["kvpair_speedup_vs_exact"] = paths["exact"]["ms_per_step"] / paths["kvpair"]["ms_per_step"]
    paths["interleaved_us_per_layer"] = {nm: mean(inter[nm]) * 1e3 / L for nm in names}
    line["value"] = paths["nectar"]["qtok_s_layer"]
    line["ms_per_step"] = total_ms / args.steps
    line["config"] = {"workload": "c5_qwen25_7b_1m_decode: Qwen2.5-7B-1M-shaped 28-layer stack, bf16, Hkv=4 Hq=28 "
                                  "d=128, 1,048,576 document keys per layer (60 GB resident), decode batch 8, "
                                  "257..384 local keys; one step = one decode step of all 28 layers through the "
                                  "Nectar (MLP 5120/3072), Quadrature (p=10,486) and exact paths; value = Nectar path",
                      "global_batch": B, "seq_len": n + cfg.T_cap, "layers": L, "parallelism": "single-gpu",
                      "document_cache": "per layer one bf16 [Hkv][n][2][d] array, K and V interleaved by key",
                      "graph": "one HIP graph per path and decode step"}
    extra["paths"] = paths
    extra["timing"] = {"ms_per_step": "all three paths (Nectar, Quadrature, exact) of one decode step of the stack",
                       "order": "each path over its own consecutive decode steps (warm-up steps, then the timed "
                                "ones); paths.interleaved_us_per_layer: the same steps with the paths interleaved",
                       "nectar_ms_per_step_median": paths["nectar"]["ms_per_step_median"],
                       "nectar_p10": paths["nectar"]["p10"], "nectar_p90": paths["nectar"]["p90"],
                       "timed_steps": args.steps, "warmup_steps": args.warmup,
                       "decode_steps": [args.warmup % cfg.decode_steps,
                                        (args.warmup + args.steps - 1) % cfg.decode_steps],
                       "clocks": clocks}
    del graphs
    return dict(extra, line=line)


def c2_layer(torch, np, nectar, configs, synth, dev, nrep=24, passes=10):
    """The Qwen3-4B-shaped decode layer (n = 61,440, 513 local keys, MLP 4608/2944):
    24 layer replicas (each its own 252 MB cache, module and local cache) rotate
    so no call reads what the previous one warmed; each measurement is one graph
    of one call per replica, replayed `passes` times.  The fused step of both
    paths, each path alone, the same step through the separate entry points, the
    components alone, and the document partial pass with its HBM roofline."""
    cfg = configs.C2
    Hkv, Hq, d, R = cfg.Hkv, cfg.Hq, cfg.d, cfg.R
    T, qoff = cfg.local_len(0), cfg.q_offset(0)

    def up(x):
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.view(torch.bfloat16) if x.dtype == np.uint16 else t).to(dev)

    q0, K0, V0 = up(synth.queries(cfg)), *(up(x) for x in synth.doc_kv(cfg))
    Kl0, Vl0 = (up(x) for x in synth.local_kv(cfg))
    P = synth.mlp_params(cfg)
    mod0 = [up(P[k]) for k in ("W1", "b1", "W2t", "b2", "Ws", "bs", "ws2", "bs2")]

    def interleaved(K_, V_):
        # one [Hkv][n][2][d] array, K and V interleaved by key, as the stack stores its caches
        kv = torch.stack((K_, V_), dim=2)
        return kv[:, :, 0], kv[:, :, 1]

    reps = [dict(q=q0.clone(), **dict(zip(("K", "V"), interleaved(K0, V0))), Kl=Kl0.clone(), Vl=Vl0.clone(),
                 mod=nectar.MLPModule(*(t.clone() for t in mod0))) for _ in range(nrep)]
    del K0, V0
    f32 = dict(dtype=torch.float32, device=dev)
    o = dict(alpha=torch.empty((R, Hq), **f32), Ax=torch.empty((R, Hq, d), **f32),
             a=torch.empty((R, Hq), **f32), Am=torch.empty((R, Hq, d), **f32),
             lam=torch.empty((R, Hq), **f32), Al=torch.empty((R, Hq, d), **f32),
             out_n=torch.empty((R, Hq, d), dtype=torch.bfloat16, device=dev), lse_n=torch.empty((R, Hq), **f32),
             out_x=torch.empty((R, Hq, d), dtype=torch.bfloat16, device=dev), lse_x=torch.empty((R, Hq), **f32))
    part_buf = torch.empty(max(16, nectar.doc_attn_partials_size(nectar.desc(R, Hq, Hkv, d, nectar.BF16), cfg.n)),
                           dtype=torch.uint8, device=dev)
    pair_out = {"out_exact": o["out_x"], "lse_exact": o["lse_x"], "alpha": o["alpha"], "A": o["Ax"],
                "out_nectar": o["out_n"], "lse_nectar": o["lse_n"], "a": o["a"], "Am": o["Am"],
                "lam": o["lam"], "Aloc": o["Al"]}
    lkw = dict(B=cfg.B, Tq=cfg.Tq, T_loc=T, q_offset=qoff)

    def fused(r, exact=True, nect=True):
        x = reps[r]
        keys = (["out_exact", "lse_exact", "alpha", "A"] if exact else []) + \
               (["out_nectar", "lse_nectar", "a", "Am"] if nect else []) + ["lam", "Aloc"]
        nectar.layer_step(x["q"], x["Kl"], x["Vl"], Hkv, k=x["K"] if exact else None, v=x["V"] if exact else None,
                          module=x["mod"] if nect else None, exact=exact, pairs=True,
                          out={k: pair_out[k] for k in keys}, **lkw)

    def doc(r):
        x = reps[r]
        nectar.doc_attn_exact(x["q"], x["K"], x["V"], Hkv, alpha_out=o["alpha"], A_out=o["Ax"])

    def module(r):
        x = reps[r]
        nectar.module_forward(x["q"], x["mod"], Hkv, a_out=o["a"], A_out=o["Am"])

    def local_nectar(r):
        x = reps[r]
        nectar.local_attn_lse(x["q"], x["Kl"], x["Vl"], Hkv, lse_out=o["lam"], A_out=o["Al"], doc_lse=o["a"],
                              doc_A=o["Am"], out=o["out_n"], out_lse=o["lse_n"], **lkw)

    def local_pair(r):
        x = reps[r]
        nectar.local_attn_lse(x["q"], x["Kl"], x["Vl"], Hkv, lse_out=o["lam"], A_out=o["Al"], **lkw)

    def merge_exact(r):
        nectar.merge(o["alpha"], o["Ax"], o["lam"], o["Al"], Hkv=Hkv, out_dtype=torch.bfloat16,
                     out=o["out_x"], lse_out=o["lse_x"])

    def doc_partial(r):
        x = reps[r]
        nectar.doc_attn_partials(x["q"], x["K"], x["V"], Hkv, partials=part_buf)

    calls = {"step": fused, "nectar": lambda r: fused(r, exact=False), "exact": lambda r: fused(r, nect=False),
             "step_unfused": lambda r: (doc(r), module(r), local_nectar(r), merge_exact(r)),
             "module": module, "local": local_pair, "merge": merge_exact, "doc": doc, "doc_partial": doc_partial}
    for fn in calls.values():
        fn(0)
    torch.cuda.synchronize()
    us = {}
    for nm, fn in calls.items():
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for r in range(nrep):
                fn(r)
        gr.replay()
        torch.cuda.synchronize()
        ev = _events(torch, passes + 1)
        ev[0].record()
        for i in range(passes):
            gr.replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) / nrep * 1e3 for i in range(passes)]
        us[nm] = {"us": sum(per) / passes, "median": _pct(per, 0.5), "p10": _pct(per, 0.1), "p90": _pct(per, 0.9)}
        del gr
    for k in ("out_n", "out_x"):
        if not torch.isfinite(o[k].float()).all():
            raise RuntimeError("non-finite output in %s" % k)
    doc_bytes = Hkv * cfg.n * 2 * d * 2
    mlp_bytes = Hkv * cfg.mlps[0].params(d) * 2
    local_bytes = cfg.B * Hkv * T * 2 * d * 2
    merge_bytes = R * Hq * (2 * 4 * (d + 1) + 2 * d + 4)
    res = {"workload": "c2_qwen3_4b_decode: Hkv=8 Hq=32 d=128 bf16, n=61,440, 513 local keys, decode batch 1, "
                       "MLP 4608/2944 GELU; %d layer replicas per graph, %d passes" % (nrep, passes),
           "step_both_paths": dict(us["step"], qtok_s_layer=R / (us["step"]["us"] * 1e-6)),
           "paths": {"nectar": dict(us["nectar"], qtok_s_layer=R / (us["nectar"]["us"] * 1e-6)),
                     "exact": dict(us["exact"], qtok_s_layer=R / (us["exact"]["us"] * 1e-6)),
                     "nectar_speedup_vs_exact": us["exact"]["us"] / us["nectar"]["us"],
                     "module_rho": cfg.rho(cfg.mlps[0].params(d))},
           "step_unfused_us": us["step_unfused"]["us"]}
    comp = {}
    for nm, nb, what in (("module", mlp_bytes, "nectar_module_forward: MLP weights of the 8 KV heads, bf16"),
                         ("local", local_bytes, "nectar_local_attn_lse: 513 causal local keys and values, bf16"),
                         ("merge", merge_bytes, "nectar_merge: two fp32 pairs in, bf16 output and fp32 LSE out")):
        u = us[nm]["us"]
        comp[nm] = {"us": u, "bytes": nb, "gbs": nb / u / 1e3, "frac": nb / u / 1e3 / HBM_PEAK_GBS, "bound": "hbm",
                    "what": what}
    res["components"] = comp
    u = us["doc_partial"]["us"]
    ach = doc_bytes / (u * 1e-6) / 1e9
    res["doc_partial_roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": ach / HBM_PEAK_GBS, "traffic": load_traffic("doc_attn_c2"),
                                   "kernel": "nectar_doc_attn_partials (attn_rows_lds, 32-key stages), %.2f us per launch, "
                                             "%d algorithmic bytes per launch" % (u, doc_bytes)}
    ue = us["doc"]["us"]
    res["exact_doc_entry_point"] = {"us": ue, "gbs": doc_bytes / (ue * 1e-6) / 1e9,
                                    "frac": doc_bytes / (ue * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                    "what": "nectar_doc_attn_exact: partial pass + combine launch"}
    del reps
    torch.cuda.empty_cache()
    return res


def profile_leg(torch, np, nectar, configs, synth, dev, args):
    """One kernel's launches alone, for counter runs: the batch-64 decode layer's
    document partial pass (LDS-staged 32-row kernel), the prefill workload's
    rho = 10 % MLP (erf GELU), or the 4B layer's document partial pass."""
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    bf = torch.bfloat16
    rn = lambda *s, std=1.0: (torch.randn(*s, generator=g, device=dev) * std).to(bf)
    n_launch = max(1, args.steps)
    if args.only == "c4_doc_partial":
        cfg = configs.C4
        q = rn(cfg.R, cfg.Hq, cfg.d)
        KV = [(x[:, :, 0], x[:, :, 1]) for x in (rn(cfg.Hkv, cfg.n, 2, cfg.d) for _ in range(2))]   # interleaved by key
        part = torch.empty(max(16, nectar.doc_attn_partials_size(nectar.desc(cfg.R, cfg.Hq, cfg.Hkv, cfg.d, nectar.BF16),
                                                                  cfg.n)), dtype=torch.uint8, device=dev)
        call = lambda i: nectar.doc_attn_partials(q, KV[i % 2][0], KV[i % 2][1], cfg.Hkv, partials=part)
        nbytes, what = cfg.Hkv * cfg.n * 2 * cfg.d * 2, "batch-64 decode layer document partial pass"
    elif args.only == "c2_doc_partial":
        cfg = configs.C2
        q = rn(cfg.R, cfg.Hq, cfg.d)
        KV = [(x[:, :, 0], x[:, :, 1]) for x in (rn(cfg.Hkv, cfg.n, 2, cfg.d) for _ in range(16))]  # interleaved by key
        part = torch.empty(max(16, nectar.doc_attn_partials_size(nectar.desc(cfg.R, cfg.Hq, cfg.Hkv, cfg.d, nectar.BF16),
                                                                  cfg.n)), dtype=torch.uint8, device=dev)
        call = lambda i: nectar.doc_attn_partials(q, KV[i % 16][0], KV[i % 16][1], cfg.Hkv, partials=part)
        nbytes, what = cfg.Hkv * cfg.n * 2 * cfg.d * 2, "4B decode layer document partial pass"
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        for _ in range(4):
            src.clone()                # calibration copies of a known size
    else:
        cfg = configs.C3
        m = cfg.mlps[1]
        q = rn(cfg.R, cfg.Hq, cfg.d)
        z = lambda *s: torch.zeros(*s, device=dev)
        mod = nectar.MLPModule(rn(cfg.Hkv, m.Ht, cfg.d, std=cfg.d ** -0.5), z(cfg.Hkv, m.Ht),
                               rn(cfg.Hkv, m.Ht, cfg.d, std=m.Ht ** -0.5), z(cfg.Hkv, cfg.d),
                               rn(cfg.Hkv, m.Hs, cfg.d, std=cfg.d ** -0.5), z(cfg.Hkv, m.Hs),
                               rn(cfg.Hkv, m.Hs, std=m.Hs ** -0.5), z(cfg.Hkv))
        a = torch.empty(cfg.R, cfg.Hq, device=dev)
        A = torch.empty(cfg.R, cfg.Hq, cfg.d, device=dev)
        call = lambda i: nectar.module_forward(q, mod, cfg.Hkv, a_out=a, A_out=A)
        nbytes = cfg.R * cfg.Hq * (4 * cfg.d * m.Ht + 2 * cfg.d * m.Hs + 2 * m.Hs)   # flops
        what = "prefill workload rho = 10 % MLP 7680/5120 (erf GELU), 458,752 rows"
    call(0)
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 2)
    e0.record()
    for i in range(n_launch):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n_launch * 1e3
    out = {"leg": args.only, "what": what, "launches": n_launch, "us_per_call": us}
    if args.only == "c3_mlp10":
        out.update(tflops=nbytes / us / 1e6, mfma_frac=nbytes / us / 1e6 / MFMA_BF16_PEAK_TFLOPS)
    else:
        out.update(gbs=nbytes / us / 1e3, frac=nbytes / us / 1e3 / HBM_PEAK_GBS)
    return out


def cpu_baseline(np, configs, synth, budget_s):
    """The fp64 oracle (test infrastructure, never tuned) on the host cores.
    `value`: the Nectar path (MLP module, local attention, merge) on one decode
    step of one layer of the 1M-token stack (8 query tokens x 28 heads),
    repeated for the budget, on up to 16 threads; the same on one thread.
    `slices`: every workload and form once -- exact document attention, each MLP
    module, the Quadrature module, local attention, merge -- on a bounded token
    sample of one layer (the oracle's cost is linear in tokens, so tokens /
    seconds is its query-tokens/s/layer)."""
    import oracle
    host = host_cpu()
    threads = max(1, min(16, host["nproc"] or 1))
    kwargs = lambda cfg, nt: dict(dt=cfg.dtype, Hq=cfg.Hq, Hkv=cfg.Hkv, threads=nt)

    def timed(fn):
        t0 = time.time()
        fn()
        return time.time() - t0

    cfg = configs.C5
    step = cfg.decode_steps - 1
    T, qoff = cfg.local_len(step), cfg.q_offset(step)
    q = synth.queries(cfg, 0, step)
    Kl, Vl = synth.local_kv(cfg)
    Klv, Vlv = (np.ascontiguousarray(x[:, :, :T]) for x in (Kl, Vl))
    P = synth.mlp_params(cfg)

    def nectar_step(nt):
        kw = kwargs(cfg, nt)
        a, Am = oracle.mlp(q, P["W1"], P["b1"], P["W2t"], P["b2"], P["Ws"], P["bs"], P["ws2"], P["bs2"], **kw)
        lam, Al = oracle.local_attn(q, Klv, Vlv, B=cfg.B, Tq=1, Tloc=T, q_offset=qoff, **kw)
        oracle.merge(a, Am, lam, Al)

    def run(nt, budget):
        n_tok, t0 = 0, time.time()
        while True:
            nectar_step(nt)
            n_tok += cfg.R
            el = time.time() - t0
            if el >= budget:
                return n_tok, el

    n_tok, el = run(threads, budget_s * 2 / 3)
    n1, el1 = run(1, budget_s / 3)
    res = {"value": n_tok / el, "unit": "query-tokens/s/layer", "cores": threads, "kind": "oracle",
           "sample": "%d tokens: decode step %d of one layer of the 1M-token stack through the Nectar path "
                     "(MLP 5120/3072, %d local keys, merge), 8 tokens x 28 heads per pass, in %.1f s"
                     % (n_tok, step, T, el),
           "single_core": {"value": n1 / el1, "sample": "%d tokens in %.1f s" % (n1, el1)}, "host": host}

    # slices of every workload and form
    slices = []

    def add(cfg_, form, ntok, secs):
        slices.append({"workload": cfg_.name, "form": form, "tokens": int(ntok), "seconds": secs,
                       "qtok_s_layer": ntok / secs, "threads": threads})

    for cfg_ in configs.BY_INDEX:
        step_ = 0 if cfg_.prefill else cfg_.decode_steps - 1
        T_, qoff_ = cfg_.local_len(step_), cfg_.q_offset(step_)
        q_ = synth.queries(cfg_, 0, step_)
        # token sample: every token (tiny workload), else one query token, else one per question up to 8
        toks = np.arange(cfg_.R, dtype=np.int32) if cfg_.R <= 16 else \
            (np.array([0], dtype=np.int32) if cfg_.prefill else np.arange(min(cfg_.B, 8), dtype=np.int32))
        kw = dict(kwargs(cfg_, threads), toks=toks)
        K_, V_ = synth.doc_kv(cfg_)
        ex_toks = toks if cfg_.n <= 131072 else toks[:1]       # the longest documents: one token
        add(cfg_, "exact", len(ex_toks), timed(lambda: oracle.doc_attn(q_, K_, V_, **dict(kw, toks=ex_toks))))
        del K_, V_
        for which, mshape in enumerate(cfg_.mlps):
            P_ = synth.mlp_params(cfg_, 0, which)
            add(cfg_, "mlp %d/%d" % (mshape.Ht, mshape.Hs), len(toks),
                timed(lambda: oracle.mlp(q_, P_["W1"], P_["b1"], P_["W2t"], P_["b2"], P_["Ws"], P_["bs"], P_["ws2"],
                                         P_["bs2"], **kw)))
        if cfg_.kv_pairs:
            W_, Z_ = synth.kv_pairs(cfg_)
            add(cfg_, "quadrature p=%d" % cfg_.kv_pairs, len(toks), timed(lambda: oracle.kvpair(q_, W_, Z_, **kw)))
        Kl_, Vl_ = synth.local_kv(cfg_)
        Klv_, Vlv_ = (np.ascontiguousarray(x[:, :, :T_]) for x in (Kl_, Vl_))
        lk = dict(B=cfg_.B, Tq=cfg_.Tq, Tloc=T_, q_offset=qoff_, **kw)
        add(cfg_, "local", len(toks), timed(lambda: oracle.local_attn(q_, Klv_, Vlv_, **lk)))
        rows = cfg_.R * cfg_.Hq
        a_, lam_ = np.zeros((cfg_.R, cfg_.Hq)), np.ones((cfg_.R, cfg_.Hq))
        A_ = np.zeros((cfg_.R, cfg_.Hq, cfg_.d))
        add(cfg_, "merge (all %d rows)" % rows, cfg_.R, timed(lambda: oracle.merge(a_, A_, lam_, A_)))
    res["slices"] = slices
    return res


MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 flop/clk, dense


def workload_layer(torch, nectar, cfg, dev):
    """One layer-step of a larger workload at its full per-layer shape: the exact
    document part alone (against its HBM or MFMA roofline), the module alone, and
    the Nectar and exact paths (document part + causal local part with the fused
    merge).  Inputs are N(0, 1) draws from a seeded device generator in the
    workload's shapes (module weights N(0, 1/fan_in)); two layer replicas when a
    layer's cache is smaller than 2 GB, so consecutive calls do not reuse a
    cache-resident copy.  Decode steps are timed as graphs, prefill eagerly."""
    g = torch.Generator(device=dev)
    g.manual_seed(1000 + cfg.seed)
    bf = torch.bfloat16
    d, Hkv, Hq, R, n = cfg.d, cfg.Hkv, cfg.Hq, cfg.R, cfg.n

    def rn(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, device=dev) * std).to(bf)

    doc_bytes = Hkv * n * 2 * d * 2
    nrep = 1 if cfg.prefill or doc_bytes >= (2 << 30) else 2
    q = rn(R, Hq, d)
    # document caches interleaved by key ([Hkv][n][2][d]), as the stack stores them
    KV = [(x[:, :, 0], x[:, :, 1]) for x in (rn(Hkv, n, 2, d) for _ in range(nrep))]
    Kl, Vl = rn(cfg.B, Hkv, cfg.T_cap, d), rn(cfg.B, Hkv, cfg.T_cap, d)
    m = cfg.mlps[-1]
    z = lambda *s: torch.zeros(*s, device=dev)
    mod = nectar.MLPModule(rn(Hkv, m.Ht, d, std=d ** -0.5), z(Hkv, m.Ht), rn(Hkv, m.Ht, d, std=m.Ht ** -0.5),
                           z(Hkv, d), rn(Hkv, m.Hs, d, std=d ** -0.5), z(Hkv, m.Hs),
                           rn(Hkv, m.Hs, std=m.Hs ** -0.5), z(Hkv))
    T, qoff = cfg.local_len(cfg.decode_steps - 1 if not cfg.prefill else 0), cfg.q_offset(cfg.decode_steps - 1 if not cfg.prefill else 0)
    f32 = dict(dtype=torch.float32, device=dev)
    al, Ax, a, Am = torch.empty((R, Hq), **f32), torch.empty((R, Hq, d), **f32), torch.empty((R, Hq), **f32), \
        torch.empty((R, Hq, d), **f32)
    out, olse = torch.empty((R, Hq, d), dtype=bf, device=dev), torch.empty((R, Hq), **f32)

    def doc(i):
        K, V = KV[i % nrep]
        nectar.doc_attn_exact(q, K, V, Hkv, alpha_out=al, A_out=Ax)

    def module(i):
        nectar.module_forward(q, mod, Hkv, a_out=a, A_out=Am)

    def local(i, x_lse, x_A):
        nectar.local_attn_lse(q, Kl, Vl, Hkv, B=cfg.B, Tq=cfg.Tq, T_loc=T, q_offset=qoff, want_pair=False,
                              doc_lse=x_lse, doc_A=x_A, out=out, out_lse=olse)

    so = {"out_exact": out, "lse_exact": olse, "out_nectar": out, "lse_nectar": olse}

    def path(i, exact, mdl):
        K, V = KV[i % nrep]
        keys = ["out_exact", "lse_exact"] if exact else ["out_nectar", "lse_nectar"]
        nectar.layer_step(q, Kl, Vl, Hkv, B=cfg.B, Tq=cfg.Tq, T_loc=T, q_offset=qoff, k=K if exact else None,
                          v=V if exact else None, module=mdl, exact=exact, out={k: so[k] for k in keys})

    parts = {"exact_doc": doc, "module": module, "local_merge": lambda i: local(i, a, Am),
             "nectar_path": lambda i: path(i, False, mod),
             "exact_path": lambda i: path(i, True, None)}
    if cfg.kv_pairs:
        kvp = nectar.KVPairModule(rn(Hkv, cfg.kv_pairs, d), rn(Hkv, cfg.kv_pairs, d))
        parts["kvpair_path"] = lambda i: path(i, False, kvp)
    for fn in parts.values():
        fn(0)
    torch.cuda.synchronize()
    us = {}
    for name, fn in parts.items():
        if cfg.prefill:
            reps = 3
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                fn(i)
            e1.record()
            torch.cuda.synchronize()
            us[name] = e0.elapsed_time(e1) / reps * 1e3
        else:
            reps = 8 * nrep
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for i in range(reps):
                    fn(i)
            gr.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(4):
                gr.replay()
            e1.record()
            torch.cuda.synchronize()
            us[name] = e0.elapsed_time(e1) / (4 * reps) * 1e3
            del gr
    if not torch.isfinite(out.float()).all():
        raise RuntimeError("non-finite output in workload %s" % cfg.name)
    res = {"layer_step": "prefill (16 x 1,024 causal tokens)" if cfg.prefill else
           "decode step %d (batch %d, %d local keys)" % (cfg.decode_steps - 1, cfg.B, T),
           "module": "MLP %d/%d" % (m.Ht, m.Hs), "us": us,
           "qtok_s_layer": {"nectar": R / (us["nectar_path"] * 1e-6), "exact": R / (us["exact_path"] * 1e-6)},
           "nectar_speedup_vs_exact": us["exact_path"] / us["nectar_path"]}
    if "kvpair_path" in us:
        res["qtok_s_layer"]["kvpair"] = R / (us["kvpair_path"] * 1e-6)
        res["kvpair_speedup_vs_exact"] = us["exact_path"] / us["kvpair_path"]
    if cfg.prefill:
        flops = R * Hq * n * 4 * d
        res["exact_doc_roofline"] = {"bound": "mfma", "tflops": flops / us["exact_doc"] / 1e6,
                                     "frac": flops / us["exact_doc"] / 1e6 / MFMA_BF16_PEAK_TFLOPS}
    else:
        res["exact_doc_roofline"] = {"bound": "hbm", "gbs": doc_bytes / us["exact_doc"] / 1e3,
                                     "frac": doc_bytes / us["exact_doc"] / 1e3 / HBM_PEAK_GBS,
                                     "bytes_per_launch": doc_bytes}
    del KV, q, Kl, Vl, mod, parts
    torch.cuda.empty_cache()
    return res


def prefill_mlp(torch, np, nectar, configs, synth, dev):
    """MFMA utilisation of the module forward at batched prefill: the 28-layer
    Qwen2.5-7B-1M-shaped stack's 16 x 1,024 query tokens x 28 heads through the
    rho = 10 % and 1 % MLPs (GELU erf form and tanh form), 4 layer replicas per graph."""
    cfg = configs.C3

    def up(x):
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.view(torch.bfloat16) if x.dtype == np.uint16 else t).to(dev)

    q = up(synth.queries(cfg))
    a = torch.empty((cfg.R, cfg.Hq), dtype=torch.float32, device=dev)
    A = torch.empty((cfg.R, cfg.Hq, cfg.d), dtype=torch.float32, device=dev)
    out = {}
    for which in (1, 0):
        P = synth.mlp_params(cfg, 0, which)
        m = cfg.mlps[which]
        flops = cfg.R * cfg.Hq * (4 * cfg.d * m.Ht + 2 * cfg.d * m.Hs + 2 * m.Hs)
        for act, name in ((nectar.GELU, "gelu_erf"), (nectar.GELU_TANH, "gelu_tanh")):
            mods = [nectar.MLPModule(*(up(P[k]) for k in ("W1", "b1", "W2t", "b2", "Ws", "bs", "ws2", "bs2")),
                                     act=act) for _ in range(4)]
            nectar.module_forward(q, mods[0], cfg.Hkv, a_out=a, A_out=A)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(8):
                    nectar.module_forward(q, mods[i % 4], cfg.Hkv, a_out=a, A_out=A)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(2):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 16
            tf = flops / ms / 1e9
            out["rho%d_%s" % (10 if which == 1 else 1, name)] = {
                "mlp": "%d/%d" % (m.Ht, m.Hs), "ms_per_layer": ms, "tflops": tf,
                "mfma_frac": tf / MFMA_BF16_PEAK_TFLOPS, "flops_per_layer": flops}
            del mods
    return out


def merge_k_prefill(torch, nectar, configs, dev, K=4):
    """HBM roofline of the K-way merge at the 16 x 1,024-token prefill shape
    (28 query heads, d = 128): K document-side fp32 pairs and the local pair in,
    the bf16 output and its log-normalizer out; N(0, 1) inputs from a seeded
    device generator."""
    cfg = configs.C3
    R, Hq, d = cfg.R, cfg.Hq, cfg.d
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    f32 = dict(dtype=torch.float32, device=dev)
    rn = lambda *s: torch.randn(*s, generator=g, **f32)
    pairs = [(rn(R, Hq), rn(R, Hq, d)) for _ in range(K)]
    lam, Al = rn(R, Hq), rn(R, Hq, d)
    out = torch.empty((R, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((R, Hq), **f32)
    call = lambda: nectar.merge_k(pairs, lam, Al, Hkv=cfg.Hkv, out_dtype=torch.bfloat16, out=out, lse_out=lse)
    call()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for _ in range(8):
            call()
    gr.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(4):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 32 * 1e3
    nbytes = R * Hq * ((K + 1) * (4 + 4 * d) + 2 * d + 4)
    del gr, pairs, lam, Al, out, lse
    torch.cuda.empty_cache()
    return {"K": K, "rows": R * Hq, "us": us, "bytes_per_launch": nbytes, "gbs": nbytes / us / 1e3,
            "frac": nbytes / us / 1e3 / HBM_PEAK_GBS, "bound": "hbm"}


def _graph_us(torch, call, reps=8, replays=4):
    call()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for _ in range(reps):
            call()
    gr.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * replays) * 1e3


def deep_modules(torch, nectar, configs, dev):
    """The deep re-injection modules of Eq. (3.6) in the depth shapes (0, 2, 3)
    and (2, 1, 2) at about 10 % capacity of the Qwen3-4B-shaped layer: the
    decode-step forward (one token x 32 heads; 16 module replicas rotate so the
    weights stream from HBM; roofline = weight bytes) and the 16 x 1,024-token
    prefill forward of the 7B-shaped layer (roofline = MFMA flops).  Weights
    N(0, 1/fan_in) from a seeded device generator, zero biases, SiLU."""
    out = {}
    g = torch.Generator(device=dev)
    g.manual_seed(79)

    def module(Hkv, d, shape):
        bf = lambda *s_, std: (torch.randn(*s_, generator=g, device=dev) * std).to(torch.bfloat16)
        layers = [(bf(Hkv, H, d, std=(d + H_in) ** -0.5), bf(Hkv, H, H_in, std=(d + H_in) ** -0.5) if H_in else None,
                   torch.zeros(Hkv, H, device=dev)) for H, H_in in shape.layers()]
        Hs, Ht = shape.last_width(1), shape.last_width(2)
        return nectar.DeepMLPModule(shape.depth, shape.width, layers, bf(Hkv, Hs, std=Hs ** -0.5),
                                    torch.zeros(Hkv, device=dev), bf(Hkv, d, Ht, std=Ht ** -0.5),
                                    torch.zeros(Hkv, d, device=dev))

    for shape in configs.DEEP_C2:
        key = "d%d%d%d" % tuple(shape.depth)
        res = {"depth": list(shape.depth), "width": list(shape.width)}
        for cfg, nrep in ((configs.C2, 16), (configs.C3, 1)):
            d, Hkv, Hq, R = cfg.d, cfg.Hkv, cfg.Hq, cfg.R
            q = torch.randn(R, Hq, d, generator=g, device=dev).to(torch.bfloat16)
            a = torch.empty(R, Hq, device=dev)
            A = torch.empty(R, Hq, d, device=dev)
            mods = [module(Hkv, d, shape) for _ in range(nrep)]
            i = [0]

            def call():
                nectar.module_forward(q, mods[i[0] % nrep], Hkv, a_out=a, A_out=A)
                i[0] += 1
            P = shape.params(d)
            if cfg.prefill:
                call()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(3):
                    call()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / 3 * 1e3
                tf = 2.0 * R * Hq * P / us / 1e6
                res["prefill_c3"] = {"us": us, "tflops": tf, "mfma_frac": tf / MFMA_BF16_PEAK_TFLOPS, "bound": "mfma",
                                     "flops": 2.0 * R * Hq * P}
            else:
                us = _graph_us(torch, call, reps=nrep, replays=4)
                nb = Hkv * P * 2
                res["decode_c2"] = {"us": us, "params_per_head": P, "rho": cfg.rho(P), "gbs": nb / us / 1e3,
                                    "frac": nb / us / 1e3 / HBM_PEAK_GBS, "bound": "hbm", "bytes": nb}
            del mods, q, a, A
            torch.cuda.empty_cache()
        out[key] = res
    return out


def train_step_bench(torch, nectar, configs, dev, tokens=1024):
    """One regression training step (loss, backward, clipping, AdamW) of the
    Qwen3-4B-shaped layer's 4608/2944 module on a batch of 1,024 query tokens x
    32 heads with fp32 targets; roofline = the algorithmic MFMA flops of its
    seven products (two first layers, the read-out, its back-propagation, three
    weight gradients; the backward's recomputed pre-activations are not
    counted).  Inputs N(0, 1) from a seeded device generator."""
    cfg = configs.C2
    m = cfg.mlps[0]
    d, Hkv, Hq = cfg.d, cfg.Hkv, cfg.Hq
    g = torch.Generator(device=dev)
    g.manual_seed(80)
    bf = lambda *s_, std=1.0: (torch.randn(*s_, generator=g, device=dev) * std).to(torch.bfloat16)
    z = lambda *s_: torch.zeros(*s_, device=dev)
    mod = nectar.MLPModule(bf(Hkv, m.Ht, d, std=d ** -0.5), z(Hkv, m.Ht), bf(Hkv, m.Ht, d, std=m.Ht ** -0.5),
                           z(Hkv, d), bf(Hkv, m.Hs, d, std=d ** -0.5), z(Hkv, m.Hs), bf(Hkv, m.Hs, std=m.Hs ** -0.5),
                           z(Hkv))
    q = bf(tokens, Hq, d)
    alpha = torch.randn(tokens, Hq, generator=g, device=dev)
    At = torch.randn(tokens, Hq, d, generator=g, device=dev) * 0.1
    theta = nectar.mlp_params_flat(mod)
    mm, vv = torch.zeros_like(theta), torch.zeros_like(theta)
    grad = torch.empty_like(theta)
    loss = torch.empty(3, device=dev)
    gn = torch.empty(2, device=dev)
    it = [0]

    def call():
        it[0] += 1
        hp = nectar.train_hparams(lr=1e-4, step=it[0], clip_norm=1.0)
        nectar.mlp_train_step(q, mod, alpha, At, Hkv, hp, theta, mm, vv, grad=grad, loss=loss, gnorm=gn)
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 10 * 1e3
    Rp = tokens * (Hq // Hkv)
    flops = Hkv * 2.0 * d * Rp * (5 * m.Ht + 2 * m.Hs)
    tf = flops / us / 1e6
    out = {"tokens": tokens, "module": "MLP %d/%d" % (m.Ht, m.Hs), "us": us, "tflops": tf,
           "mfma_frac": tf / MFMA_BF16_PEAK_TFLOPS, "bound": "mfma", "flops": flops,
           "loss_after": float(loss[0]), "params": int(theta.numel())}
    del mod, q, alpha, At, theta, mm, vv, grad
    torch.cuda.empty_cache()
    return out


def fit_metrics_prefill(torch, nectar, configs, dev):
    """HBM roofline of the fit metrics (squared errors and the RTE summand of a
    module pair against the exact pair, with per-KV-head sums) at the
    16 x 1,024-token prefill shape: q (bf16), both pairs (fp32) in, the per-row
    values out."""
    cfg = configs.C3
    R, Hq, d = cfg.R, cfg.Hq, cfg.d
    g = torch.Generator(device=dev)
    g.manual_seed(78)
    f32 = dict(dtype=torch.float32, device=dev)
    rn = lambda *s: torch.randn(*s, generator=g, **f32)
    q = rn(R, Hq, d).to(torch.bfloat16)
    a, alpha, A, Aex = rn(R, Hq), rn(R, Hq), rn(R, Hq, d), rn(R, Hq, d)
    row = torch.empty((R, Hq, 3), **f32)
    head = torch.empty((cfg.Hkv, 3), dtype=torch.float64, device=dev)
    us = _graph_us(torch, lambda: nectar.fit_metrics(q, a, A, alpha, Aex, cfg.Hkv, row_out=row, head_out=head))
    nbytes = R * Hq * (2 * d + 2 * 4 * d + 2 * 4 + 3 * 4)
    del q, a, alpha, A, Aex, row, head
    torch.cuda.empty_cache()
    return {"rows": R * Hq, "us": us, "bytes_per_call": nbytes, "gbs": nbytes / us / 1e3,
            "frac": nbytes / us / 1e3 / HBM_PEAK_GBS, "bound": "hbm",
            "what": "nectar_fit_metrics: row pass + per-KV-head fp64 sums (three launches)"}


def gpu_clocks():
    """The current shader, memory and fabric clock levels of the device as the
    driver lists them (the entries marked current), read while work runs."""
    import glob
    out = {}
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_*clk")):
        try:
            with open(f) as fh:
                cur = [ln.split(":", 1)[1].strip(" *\n") for ln in fh if ln.rstrip().endswith("*")]
        except OSError:
            continue
        if cur:
            out["%s %s" % (f.split("/")[4], os.path.basename(f)[7:])] = cur[0]
    if not out:
        import subprocess
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=30)
            for card, kv in json.loads(r.stdout).items():
                for k, v in kv.items():
                    if "clk" in k.lower():
                        out["%s %s" % (card, k.strip(" :"))] = v
        except (OSError, ValueError, AttributeError, subprocess.SubprocessError):
            pass
    return out or None


def host_cpu():
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"nproc": usable, "cpu_count": os.cpu_count(), "model": model}


if __name__ == "__main__":
    main()
