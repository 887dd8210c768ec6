"""GPU parity on the three large workloads at their full per-layer sizes.

Each layer's whole step runs on the GPU (every token), twice: through the
separate entry points (document pair, module pair, local attention with the
fused merge) and through ``nectar_layer_step`` called exactly as the benchmark
times it (the same output set, the automatic split plan, one call per path).
The fp64 oracle checks a sample of tokens that the CPU finishes in seconds,
covering every KV head and query head, the first and last tokens of the first
and last questions, and first/last decode steps or layers:

* the 28-layer Qwen2.5-7B-1M-shaped prefill (n = 131,072, 16 x 1,024 causal
  tokens, both MLP capacities) at layers 0, 13 and 27,
* the 32-layer Llama-3.1-8B-shaped decode (n = 262,144, batch 64: 16 of the 64
  questions) at layers {0, 31} x decode steps {0, 127},
* the 28-layer 1M-token decode (n = 1,048,576, batch 8: MLP, Quadrature, exact)
  at layers {0, 27} x decode steps {0, 127}.
"""
import functools

import numpy as np
import torch
import pytest

import oracle
from helpers import ATOL_LSE_BF16, ATOL_OUT_BF16, REL_L2_BF16, check, dev, host
from learned_kv_cache_02_amd import configs, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nx(gpu):
    from learned_kv_cache_02_amd import nectar
    return nectar


@functools.lru_cache(maxsize=1)
def _doc(cfg, layer):
    # the document cache depends on the layer only: shared by the decode steps of one layer
    return synth.doc_kv(cfg, layer)


def _mlp_dev(nx, P):
    return nx.MLPModule(*(dev(P[k]) for k in ("W1", "b1", "W2t", "b2", "Ws", "bs", "ws2", "bs2")))


def _check_pair(name, got_a, got_A, ref_a, ref_A):
    check(name + " lse", got_a, ref_a, ATOL_LSE_BF16)
    check(name + " read-out", got_A, ref_A, ATOL_OUT_BF16, REL_L2_BF16)


def _check_merged(name, out, lse, ref_out, ref_lse):
    check(name + " merged out", out, ref_out, ATOL_OUT_BF16, REL_L2_BF16)
    check(name + " merged lse", lse, ref_lse, ATOL_LSE_BF16)


def _layer(nx, cfg, layer, step, toks, modules=(), kv_pairs=False):
    """Run the layer on the GPU through the separate entry points and through the
    layer step as timed, and compare sampled tokens with the oracle."""
    print("case %s layer %d step %d (%d sampled tokens)" % (cfg.name, layer, step, len(toks)), flush=True)
    q = synth.queries(cfg, layer, step)
    K, V = _doc(cfg, layer)
    Kl, Vl = synth.local_kv(cfg, layer)
    T, qoff = cfg.local_len(step), cfg.q_offset(step)
    qd, Kd, Vd, Kld, Vld = dev(q), dev(K), dev(V), dev(Kl), dev(Vl)
    kw = dict(dt="bf16", Hq=cfg.Hq, Hkv=cfg.Hkv, toks=toks, threads=16)
    skw = dict(B=cfg.B, Tq=cfg.Tq, T_loc=T, q_offset=qoff)
    pick = lambda *ts: [host(t)[toks] for t in ts]

    # oracle: document pair, local pair, their merge (= full attention, App. B)
    ea, eA = oracle.doc_attn(q, K, V, **kw)
    Klv, Vlv = (np.ascontiguousarray(x[:, :, :T]) for x in (Kl, Vl))
    el, eAl = oracle.local_attn(q, Klv, Vlv, B=cfg.B, Tq=cfg.Tq, Tloc=T, q_offset=qoff, **kw)
    eo, e_lse = oracle.merge(ea, eA, el, eAl)

    # separate entry points
    alpha, A = nx.doc_attn_exact(qd, Kd, Vd, cfg.Hkv)
    lam, Al, out_x, lse_x = nx.local_attn_lse(qd, Kld, Vld, cfg.Hkv, doc_lse=alpha, doc_A=A, **skw)
    alpha, A, lam, Al, out_x, lse_x = pick(alpha, A, lam, Al, out_x, lse_x)
    _check_pair("exact doc", alpha, A, ea, eA)
    _check_pair("local", lam, Al, el, eAl)
    _check_merged("exact", out_x, lse_x, eo, e_lse)

    # the exact path as the benchmark times it: the document cache as one array with
    # K and V interleaved by key; merged output and lse only
    kv = torch.stack((Kd, Vd), dim=2)
    del Kd, Vd
    Ki, Vi = kv[:, :, 0], kv[:, :, 1]
    st = nx.layer_step(qd, Kld, Vld, cfg.Hkv, k=Ki, v=Vi, module=None, exact=True, **skw)
    _check_merged("layer step exact path", *pick(st["out_exact"], st["lse_exact"]), eo, e_lse)
    # ... and with every pair requested
    st = nx.layer_step(qd, Kld, Vld, cfg.Hkv, k=Ki, v=Vi, module=None, exact=True, pairs=True, **skw)
    _check_pair("layer step alpha/A", *pick(st["alpha"], st["A"]), ea, eA)
    _check_pair("layer step local", *pick(st["lam"], st["Aloc"]), el, eAl)
    del kv, Ki, Vi, st

    for which in modules:
        P = synth.mlp_params(cfg, layer, which)
        mod = _mlp_dev(nx, P)
        em, eAm = oracle.mlp(q, P["W1"], P["b1"], P["W2t"], P["b2"], P["Ws"], P["bs"], P["ws2"], P["bs2"], **kw)
        eon, eln = oracle.merge(em, eAm, el, eAl)
        name = "mlp %d/%d" % (P["Ht"], P["Hs"])
        a, Am = nx.module_forward(qd, mod, cfg.Hkv)
        out_n, lse_n = nx.local_attn_lse(qd, Kld, Vld, cfg.Hkv, doc_lse=a, doc_A=Am, want_pair=False, **skw)
        a, Am, out_n, lse_n = pick(a, Am, out_n, lse_n)
        _check_pair(name, a, Am, em, eAm)
        _check_merged("nectar " + name, out_n, lse_n, eon, eln)
        # the Nectar path as timed, then with its pairs
        st = nx.layer_step(qd, Kld, Vld, cfg.Hkv, module=mod, exact=False, **skw)
        _check_merged("layer step nectar path " + name, *pick(st["out_nectar"], st["lse_nectar"]), eon, eln)
        st = nx.layer_step(qd, Kld, Vld, cfg.Hkv, module=mod, exact=False, pairs=True, **skw)
        _check_pair("layer step " + name, *pick(st["a"], st["Am"]), em, eAm)
        _check_pair("layer step local (nectar)", *pick(st["lam"], st["Aloc"]), el, eAl)
        del mod, st

    if kv_pairs:
        W, Z = synth.kv_pairs(cfg, layer)
        kvp = nx.KVPairModule(dev(W), dev(Z))
        ek, eAk = oracle.kvpair(q, W, Z, **kw)
        eok, elk = oracle.merge(ek, eAk, el, eAl)
        a, Aq = nx.module_forward(qd, kvp, cfg.Hkv)
        out_n, lse_n = nx.local_attn_lse(qd, Kld, Vld, cfg.Hkv, doc_lse=a, doc_A=Aq, want_pair=False, **skw)
        a, Aq, out_n, lse_n = pick(a, Aq, out_n, lse_n)
        _check_pair("kv pairs p=%d" % cfg.kv_pairs, a, Aq, ek, eAk)
        _check_merged("kv-pair", out_n, lse_n, eok, elk)
        st = nx.layer_step(qd, Kld, Vld, cfg.Hkv, module=kvp, exact=False, **skw)
        _check_merged("layer step kv-pair path", *pick(st["out_nectar"], st["lse_nectar"]), eok, elk)
        st = nx.layer_step(qd, Kld, Vld, cfg.Hkv, module=kvp, exact=False, pairs=True, **skw)
        _check_pair("layer step kv pairs", *pick(st["a"], st["Am"]), ek, eAk)


def _prefill_tokens(cfg, k=60, seed=0):
    g = np.random.default_rng(seed)
    edge = [0, 1, cfg.Tq - 1, (cfg.B - 1) * cfg.Tq, cfg.R - 1]
    rest = g.choice(np.arange(cfg.R), size=k - len(edge), replace=False)
    return np.unique(np.concatenate([edge, rest])).astype(np.int32)


@pytest.mark.parametrize("layer,mods", [(0, (0, 1)), (13, (1,)), (27, (0, 1))])
def test_qwen25_7b_prefill_layer(nx, layer, mods):
    cfg = configs.C3
    _layer(nx, cfg, layer, 0, _prefill_tokens(cfg, seed=layer), modules=mods)


# 16 of the 64 questions (one query token each): both ends and every fourth-ish in between
C4_QUESTIONS = np.array([0, 1, 5, 9, 14, 17, 22, 28, 31, 32, 38, 45, 50, 57, 62, 63], dtype=np.int32)


@pytest.mark.parametrize("layer,step", [(0, 0), (0, 127), (31, 0), (31, 127)])
def test_llama31_8b_decode_layer(nx, layer, step):
    _layer(nx, configs.C4, layer, step, C4_QUESTIONS, modules=(0,))


@pytest.mark.parametrize("layer,step", [(0, 0), (0, 127), (27, 0), (27, 127)])
def test_qwen25_7b_1m_decode_layer(nx, layer, step):
    cfg = configs.C5
    _layer(nx, cfg, layer, step, np.arange(cfg.B, dtype=np.int32), modules=(0,), kv_pairs=True)
