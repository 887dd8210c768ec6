#!/usr/bin/env python3
"""Benchmark of the Nectar attention hot path on one MI355X.

Workload: the Qwen3-4B-shaped decode layer (8 KV heads, 32 query heads, d=128,
bf16; document n = 61,440 keys; local cache 512 prompt tokens + the decode
token; Nectar MLP 128->4608->128 target and 128->2944->1 score per KV head,
GELU).  A step is one decode step of one layer through the whole hot path:

  exact document attention (alpha, A) over the 61,440-key cache,
  the MLP module forward (a, A_theta),
  causal local attention over the 513 local keys (lambda, A_local),
  and both merges: the module pair with the local pair (the Nectar output) and
  the exact pair with the local pair (the exact output),

through the fused layer-step entry point (the document, local and module
partials in one launch, then one finishing launch that writes every pair and
both outputs).  The same step through the four separate entry points is timed
too (`paths.step_unfused_us`).

Every step reads a distinct layer replica (its own document cache, module and
local cache), so consecutive steps never hit a cache the previous step
warmed; the replicas together exceed the 256 MB Infinity Cache many times.
Inputs are resident in HBM before timing.  The launches of one pass over all
replicas (one step per replica, like a decode step through a stack of that
many layers) are captured once in a HIP graph and replayed; timing uses HIP
events on the replay stream around K steps (K rounded up to whole passes),
bracketed by synchronizations.

Prints one JSON line.  `value` is query-tokens/s/layer of the whole step (mean
over the timed steps); `timing` gives the median and 10th/90th percentiles of
the per-pass step times and the device clocks read while the step runs;
`paths` gives the Nectar and exact paths timed alone, `components` the module,
local attention and merge alone against their HBM rooflines; `roofline` covers
the dominant kernel (exact document attention, HBM-bound); `cpu_baseline` times
the fp64 CPU oracle on a bounded sample of the same step, multithreaded and on
one thread, with the host's CPU model.
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
SOURCES_FOR_TRAFFIC = ["learned_kv_cache_02_amd/csrc/" + f for f in
                       ("attn.hip", "attn_body.hpp", "attn_common.hpp", "device_common.hpp", "kernels.hpp")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=24)
    ap.add_argument("--replicas", type=int, default=24)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle sample budget (0: skip)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--only", choices=["step", "exact", "nectar", "doc", "doc_partial"], default=None,
                    help="time only one graph (for profiling runs)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the per-layer timings of the three larger workloads")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the batched-prefill MLP measurement")
    return ap.parse_args()


def source_hash():
    h = hashlib.sha256()
    for f in SOURCES_FOR_TRAFFIC:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from learned_kv_cache_02_amd import configs, nectar, synth

    cfg = configs.C2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    NREP = args.replicas

    def up(x):
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.view(torch.bfloat16) if x.dtype == np.uint16 else t).to(dev)

    t0 = time.time()
    q_h = synth.queries(cfg)
    K_h, V_h = synth.doc_kv(cfg)
    Kl_h, Vl_h = synth.local_kv(cfg)
    P_h = synth.mlp_params(cfg)
    gen_s = time.time() - t0
    print("generated inputs in %.1fs" % gen_s, file=sys.stderr, flush=True)

    q0, K0, V0, Kl0, Vl0 = up(q_h), up(K_h), up(V_h), up(Kl_h), up(Vl_h)
    mod0 = [up(P_h[k]) for k in ("W1", "b1", "W2t", "b2", "Ws", "bs", "ws2", "bs2")]
    reps = []
    for r in range(NREP):
        reps.append(dict(q=q0.clone(), K=K0.clone(), V=V0.clone(), Kl=Kl0.clone(), Vl=Vl0.clone(),
                         mod=nectar.MLPModule(*(t.clone() for t in mod0))))
    del K0, V0
    torch.cuda.synchronize()

    Hkv, Hq, d, R = cfg.Hkv, cfg.Hq, cfg.d, cfg.R
    T, qoff = cfg.local_len(0), cfg.q_offset(0)
    f32 = dict(dtype=torch.float32, device=dev)
    o = dict(alpha=torch.empty((R, Hq), **f32), Ax=torch.empty((R, Hq, d), **f32),
             a=torch.empty((R, Hq), **f32), Am=torch.empty((R, Hq, d), **f32),
             lam=torch.empty((R, Hq), **f32), Al=torch.empty((R, Hq, d), **f32),
             out_n=torch.empty((R, Hq, d), dtype=torch.bfloat16, device=dev), lse_n=torch.empty((R, Hq), **f32),
             out_x=torch.empty((R, Hq, d), dtype=torch.bfloat16, device=dev), lse_x=torch.empty((R, Hq), **f32))

    def doc(r):
        x = reps[r]
        nectar.doc_attn_exact(x["q"], x["K"], x["V"], Hkv, alpha_out=o["alpha"], A_out=o["Ax"])

    part_dsc = nectar.desc(R, Hq, Hkv, d, nectar.BF16)
    part_buf = torch.empty(max(16, nectar.doc_attn_partials_size(part_dsc, cfg.n)), dtype=torch.uint8, device=dev)

    def doc_partial(r):
        # the split-K partial pass alone: the dominant kernel of the step
        x = reps[r]
        nectar.doc_attn_partials(x["q"], x["K"], x["V"], Hkv, partials=part_buf)

    def module(r):
        x = reps[r]
        nectar.module_forward(x["q"], x["mod"], Hkv, a_out=o["a"], A_out=o["Am"])

    def local_nectar(r):
        x = reps[r]
        nectar.local_attn_lse(x["q"], x["Kl"], x["Vl"], Hkv, B=cfg.B, Tq=cfg.Tq, T_loc=T, q_offset=qoff,
                              lse_out=o["lam"], A_out=o["Al"], doc_lse=o["a"], doc_A=o["Am"],
                              out=o["out_n"], out_lse=o["lse_n"])

    def local_pair(r):
        x = reps[r]
        nectar.local_attn_lse(x["q"], x["Kl"], x["Vl"], Hkv, B=cfg.B, Tq=cfg.Tq, T_loc=T, q_offset=qoff,
                              lse_out=o["lam"], A_out=o["Al"])

    def merge_exact(r):
        nectar.merge(o["alpha"], o["Ax"], o["lam"], o["Al"], Hkv=Hkv, out_dtype=torch.bfloat16,
                     out=o["out_x"], lse_out=o["lse_x"])

    pair_out = {"out_exact": o["out_x"], "lse_exact": o["lse_x"], "alpha": o["alpha"], "A": o["Ax"],
                "out_nectar": o["out_n"], "lse_nectar": o["lse_n"], "a": o["a"], "Am": o["Am"],
                "lam": o["lam"], "Aloc": o["Al"]}

    def fused(r, exact=True, nect=True):
        x = reps[r]
        keys = (["out_exact", "lse_exact", "alpha", "A"] if exact else []) + \
               (["out_nectar", "lse_nectar", "a", "Am"] if nect else []) + ["lam", "Aloc"]
        nectar.layer_step(x["q"], x["Kl"], x["Vl"], Hkv, B=cfg.B, Tq=cfg.Tq, T_loc=T, q_offset=qoff,
                          k=x["K"] if exact else None, v=x["V"] if exact else None,
                          module=x["mod"] if nect else None, exact=exact, pairs=True,
                          out={k: pair_out[k] for k in keys})

    steps = {
        # the whole step of both paths through the fused layer-step entry point
        "step": lambda r: fused(r),
        "nectar": lambda r: fused(r, exact=False),
        "exact": lambda r: fused(r, nect=False),
        "doc": lambda r: doc(r),
        "doc_partial": lambda r: doc_partial(r),
        # the same step through the four separate entry points (seven launches)
        "step_unfused": lambda r: (doc(r), module(r), local_nectar(r), merge_exact(r)),
        # the components alone
        "module": lambda r: module(r),
        "local": lambda r: local_pair(r),
        "merge": lambda r: merge_exact(r),
    }
    names = [args.only] if args.only else ["step", "nectar", "exact", "doc", "doc_partial", "step_unfused",
                                           "module", "local", "merge"]

    # warm every call once (allocates the binding's cached workspace outside capture)
    for fn in steps.values():
        fn(0)
    torch.cuda.synchronize()

    graphs = {}
    if not args.no_graph:
        for nm in names:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for r in range(NREP):
                    steps[nm](r)
            graphs[nm] = g
        torch.cuda.synchronize()

    passes = max(1, -(-args.steps // NREP))
    wpasses = max(1, -(-args.warmup // NREP))
    n_steps, n_warm = passes * NREP, wpasses * NREP

    def one_pass(nm):
        if args.no_graph:
            for r in range(NREP):
                steps[nm](r)
        else:
            graphs[nm].replay()

    def timed(nm):
        for _ in range(wpasses):
            one_pass(nm)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(passes):
            one_pass(nm)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n_steps   # ms per step

    ms = {nm: timed(nm) for nm in names}

    # spread of the step time: each pass of the step graph timed on its own
    spread = None
    if "step" in ms and not args.no_graph:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(passes + 1)]
        ev[0].record()
        for i in range(passes):
            one_pass("step")
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = sorted(ev[i].elapsed_time(ev[i + 1]) / NREP * 1e3 for i in range(passes))
        pick = lambda f: per[min(len(per) - 1, int(round(f * (len(per) - 1))))]
        spread = {"us_per_step_median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9), "passes": passes,
                  "steps_per_pass": NREP}
        # the clocks while the step runs: enqueue about a second of passes, then read them
        for _ in range(max(1, int(1.0 / (ms["step"] * 1e-3 * NREP)))):
            one_pass("step")
        spread["clocks"] = gpu_clocks()
        torch.cuda.synchronize()

    # Correctness spot check of the timed outputs against the oracle is the job of
    # the test suite; here only finite outputs are asserted.
    for k in ("out_n", "out_x"):
        if not torch.isfinite(o[k].float()).all():
            raise RuntimeError("non-finite output in %s" % k)

    layer_tokens = R * 1   # one layer per step
    doc_bytes = Hkv * cfg.n * 2 * d * 2
    mlp_bytes = Hkv * cfg.mlps[0].params(d) * 2
    res = {
        "metric": "query-tokens/s/layer, Nectar vs exact cache attn; % of HBM / MFMA roofline",
        "unit": "query-tokens/s/layer",
        "higher_is_better": True,
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": n_warm,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    if "step" in ms:
        res["value"] = layer_tokens / (ms["step"] / 1e3)
        res["ms_per_step"] = ms["step"]
    res["config"] = {"workload": "%s: Hkv=8 Hq=32 d=128 bf16, n=61440 document keys, 513 local keys, "
                                 "decode batch 1, MLP 4608/2944 GELU; one layer replica per step, %d replicas"
                                 % (cfg.name, NREP),
                     "global_batch": cfg.B, "seq_len": cfg.n + T, "parallelism": "single-gpu",
                     "graph": not args.no_graph}
    paths = {}
    for nm in ("nectar", "exact"):
        if nm in ms:
            paths[nm] = {"qtok_s_layer": layer_tokens / (ms[nm] / 1e3), "us_per_layer": ms[nm] * 1e3}
    if "nectar" in ms and "exact" in ms:
        paths["nectar_speedup_vs_exact"] = ms["exact"] / ms["nectar"]
        paths["module_rho"] = cfg.rho(cfg.mlps[0].params(d))
    if "step_unfused" in ms:
        paths["step_unfused_us"] = ms["step_unfused"] * 1e3
    res["paths"] = paths
    if spread:
        res["timing"] = spread
    local_bytes = cfg.B * Hkv * T * 2 * d * 2
    merge_bytes = R * Hq * (2 * 4 * (d + 1) + 2 * d + 4)
    comp = {}
    for nm, nb, what in (("module", mlp_bytes, "nectar_module_forward: MLP weights of the 8 KV heads, bf16"),
                         ("local", local_bytes, "nectar_local_attn_lse: 513 causal local keys and values, bf16"),
                         ("merge", merge_bytes, "nectar_merge: two fp32 pairs in, bf16 output and fp32 LSE out")):
        if nm in ms:
            us_c = ms[nm] * 1e3
            comp[nm] = {"us": us_c, "bytes": nb, "gbs": nb / us_c / 1e3, "frac": nb / us_c / 1e3 / HBM_PEAK_GBS,
                        "bound": "hbm", "what": what}
    if comp:
        res["components"] = comp
    if "doc_partial" in ms:
        us = ms["doc_partial"] * 1e3
        ach = doc_bytes / (us * 1e-6) / 1e9
        traffic = None
        tf = os.path.join(ROOT, "profiles", "traffic_doc_attn_c2.json")
        if os.path.exists(tf):
            with open(tf) as fh:
                tj = json.load(fh)
            if tj.get("source_hash") == source_hash():
                traffic = tj.get("hbm_bytes_per_launch")
        res["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBS, "traffic": traffic,
                           "kernel": "split-K partial pass of the exact document attention "
                                     "(nectar_doc_attn_partials: attn_partial_mfma, one launch), %.2f us per launch, "
                                     "%d algorithmic bytes per launch" % (us, doc_bytes)}
    if "doc" in ms:
        us_e = ms["doc"] * 1e3
        res["exact_doc_entry_point"] = {"us": us_e, "gbs": doc_bytes / (us_e * 1e-6) / 1e9,
                                        "frac": doc_bytes / (us_e * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                        "what": "nectar_doc_attn_exact: partial pass + combine launch"}

    if args.only is None and not (args.no_prefill and args.no_workloads):
        del reps, graphs
        torch.cuda.empty_cache()
    if not args.no_prefill and args.only is None:
        res["prefill_mlp"] = prefill_mlp(torch, np, nectar, configs, synth, dev)
        res["merge_k"] = merge_k_prefill(torch, nectar, configs, dev)
        res["fit_metrics"] = fit_metrics_prefill(torch, nectar, configs, dev)
        res["deep_modules"] = deep_modules(torch, nectar, configs, dev)
        res["train_step"] = train_step_bench(torch, nectar, configs, dev)
    if not args.no_workloads and args.only is None:
        res["workloads"] = {c.name: workload_layer(torch, nectar, c, dev) for c in (configs.C4, configs.C5, configs.C3)}

    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(cfg, q_h, K_h, V_h, Kl_h, Vl_h, P_h, args.cpu_seconds)
    print(json.dumps(res), flush=True)


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
    KV = [(rn(Hkv, n, d), rn(Hkv, n, d)) for _ in range(nrep)]
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
    32 heads with fp32 targets; roofline = the MFMA flops of its seven products
    (two first layers, the read-out, its back-propagation, three weight
    gradients).  Inputs N(0, 1) from a seeded device generator."""
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


def cpu_baseline(cfg, q, K, V, Kl, Vl, P, budget_s):
    """The fp64 oracle on the same step (both paths, one token), repeated until
    the time budget is used; tokens per second per layer.  Two thirds of the
    budget go to a run on up to 16 threads (the reported value), the rest to a
    single-thread run."""
    import numpy as np

    import oracle
    host = host_cpu()
    threads = max(1, min(16, host["nproc"] or 1))
    T = cfg.local_len(0)
    Klv, Vlv = (np.ascontiguousarray(x[:, :, :T]) for x in (Kl, Vl))

    def run(nthreads, budget):
        kw = dict(dt="bf16", Hq=cfg.Hq, Hkv=cfg.Hkv, threads=nthreads)
        n_tok = 0
        t0 = time.time()
        while True:
            alpha, A = oracle.doc_attn(q, K, V, **kw)
            a, Am = oracle.mlp(q, P["W1"], P["b1"], P["W2t"], P["b2"], P["Ws"], P["bs"], P["ws2"], P["bs2"], **kw)
            lam, Al = oracle.local_attn(q, Klv, Vlv, B=cfg.B, Tq=cfg.Tq, Tloc=T, q_offset=cfg.q_offset(0), **kw)
            oracle.merge(a, Am, lam, Al)
            oracle.merge(alpha, A, lam, Al)
            n_tok += cfg.R
            el = time.time() - t0
            if el >= budget:
                return n_tok, el

    n_tok, el = run(threads, budget_s * 2 / 3)
    n1, el1 = run(1, budget_s / 3)
    return {"value": n_tok / el, "unit": "query-tokens/s/layer", "cores": threads, "kind": "oracle",
            "sample": "%d decode steps of the same layer (exact + Nectar paths, 1 query token x 32 heads "
                      "each) in %.1f s" % (n_tok, el),
            "single_core": {"value": n1 / el1, "sample": "%d steps in %.1f s" % (n1, el1)}, "host": host}


if __name__ == "__main__":
    main()
