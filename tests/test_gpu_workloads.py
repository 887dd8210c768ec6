"""GPU parity on the three large workloads at their full per-layer sizes.

Each layer's whole step runs on the GPU (every token); the fp64 oracle checks a
sample of tokens that the CPU finishes in seconds, covering every KV head and
query head, the first and last tokens of the first and last questions, and
first/last decode steps or layers:

* the 28-layer Qwen2.5-7B-1M-shaped prefill (n = 131,072, 16 x 1,024 causal
  tokens, both MLP capacities),
* the 32-layer Llama-3.1-8B-shaped decode (n = 262,144, batch 64),
* the 28-layer 1M-token decode (n = 1,048,576, batch 8: MLP, Quadrature, exact).
"""
import numpy as np
import pytest

import oracle
from helpers import ATOL_LSE_BF16, ATOL_OUT_BF16, REL_L2_BF16, check, dev, host
from learned_kv_cache_02_amd import configs, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nx(gpu):
    from learned_kv_cache_02_amd import nectar
    return nectar


def _mlp_dev(nx, P):
    return nx.MLPModule(*(dev(P[k]) for k in ("W1", "b1", "W2t", "b2", "Ws", "bs", "ws2", "bs2")))


def _check_pair(name, got_a, got_A, ref_a, ref_A):
    check(name + " lse", got_a, ref_a, ATOL_LSE_BF16)
    check(name + " read-out", got_A, ref_A, ATOL_OUT_BF16, REL_L2_BF16)


def _layer(nx, cfg, layer, step, toks, modules=(), kv_pairs=False):
    """Run the layer step on the GPU and compare sampled tokens with the oracle."""
    print("case %s layer %d step %d (%d sampled tokens)" % (cfg.name, layer, step, len(toks)), flush=True)
    q = synth.queries(cfg, layer, step)
    K, V = synth.doc_kv(cfg, layer)
    Kl, Vl = synth.local_kv(cfg, layer)
    T, qoff = cfg.local_len(step), cfg.q_offset(step)
    qd, Kd, Vd, Kld, Vld = dev(q), dev(K), dev(V), dev(Kl), dev(Vl)
    kw = dict(dt="bf16", Hq=cfg.Hq, Hkv=cfg.Hkv, toks=toks, threads=16)

    alpha, A = nx.doc_attn_exact(qd, Kd, Vd, cfg.Hkv)
    lam, Al, out_x, lse_x = nx.local_attn_lse(qd, Kld, Vld, cfg.Hkv, B=cfg.B, Tq=cfg.Tq, T_loc=T,
                                              q_offset=qoff, doc_lse=alpha, doc_A=A)
    alpha, A, lam, Al, out_x, lse_x = (host(t)[toks] for t in (alpha, A, lam, Al, out_x, lse_x))
    del Kd, Vd
    ea, eA = oracle.doc_attn(q, K, V, **kw)
    _check_pair("exact doc", alpha, A, ea, eA)
    Klv, Vlv = (np.ascontiguousarray(x[:, :, :T]) for x in (Kl, Vl))
    el, eAl = oracle.local_attn(q, Klv, Vlv, B=cfg.B, Tq=cfg.Tq, Tloc=T, q_offset=qoff, **kw)
    _check_pair("local", lam, Al, el, eAl)
    eo, e_lse = oracle.merge(ea, eA, el, eAl)
    check("exact merged out", out_x, eo, ATOL_OUT_BF16, REL_L2_BF16)
    check("exact merged lse", lse_x, e_lse, ATOL_LSE_BF16)
    del K, V

    for which in modules:
        P = synth.mlp_params(cfg, layer, which)
        a, Am = nx.module_forward(qd, _mlp_dev(nx, P), cfg.Hkv)
        out_n, lse_n = nx.local_attn_lse(qd, Kld, Vld, cfg.Hkv, B=cfg.B, Tq=cfg.Tq, T_loc=T, q_offset=qoff,
                                         doc_lse=a, doc_A=Am, want_pair=False)
        a, Am, out_n, lse_n = (host(t)[toks] for t in (a, Am, out_n, lse_n))
        em, eAm = oracle.mlp(q, P["W1"], P["b1"], P["W2t"], P["b2"], P["Ws"], P["bs"], P["ws2"], P["bs2"], **kw)
        _check_pair("mlp %d/%d" % (P["Ht"], P["Hs"]), a, Am, em, eAm)
        eo, e_lse = oracle.merge(em, eAm, el, eAl)
        check("nectar merged out", out_n, eo, ATOL_OUT_BF16, REL_L2_BF16)
        check("nectar merged lse", lse_n, e_lse, ATOL_LSE_BF16)

    if kv_pairs:
        W, Z = synth.kv_pairs(cfg, layer)
        a, Aq = nx.module_forward(qd, nx.KVPairModule(dev(W), dev(Z)), cfg.Hkv)
        out_n, lse_n = nx.local_attn_lse(qd, Kld, Vld, cfg.Hkv, B=cfg.B, Tq=cfg.Tq, T_loc=T, q_offset=qoff,
                                         doc_lse=a, doc_A=Aq, want_pair=False)
        a, Aq, out_n, lse_n = (host(t)[toks] for t in (a, Aq, out_n, lse_n))
        ek, eAk = oracle.kvpair(q, W, Z, **kw)
        _check_pair("kv pairs p=%d" % cfg.kv_pairs, a, Aq, ek, eAk)
        eo, e_lse = oracle.merge(ek, eAk, el, eAl)
        check("kv-pair merged out", out_n, eo, ATOL_OUT_BF16, REL_L2_BF16)


def _prefill_tokens(cfg, k=60, seed=0):
    g = np.random.default_rng(seed)
    edge = [0, cfg.Tq - 1, (cfg.B - 1) * cfg.Tq, cfg.R - 1]
    rest = g.choice(np.arange(cfg.R), size=k - len(edge), replace=False)
    return np.unique(np.concatenate([edge, rest])).astype(np.int32)


@pytest.mark.parametrize("layer", [0, 27])
def test_qwen25_7b_prefill_layer(nx, layer):
    cfg = configs.C3
    _layer(nx, cfg, layer, 0, _prefill_tokens(cfg, seed=layer), modules=(0, 1) if layer == 0 else (1,))


@pytest.mark.parametrize("layer,step", [(0, 0), (31, 127)])
def test_llama31_8b_decode_layer(nx, layer, step):
    cfg = configs.C4
    toks = np.array([0, 1, 17, 31, 32, 45, 62, 63], dtype=np.int32)   # questions (one token each)
    _layer(nx, cfg, layer, step, toks, modules=(0,))


@pytest.mark.parametrize("layer,step", [(0, 0), (27, 127)])
def test_qwen25_7b_1m_decode_layer(nx, layer, step):
    cfg = configs.C5
    toks = np.arange(cfg.B, dtype=np.int32)
    _layer(nx, cfg, layer, step, toks, modules=(0,), kv_pairs=True)
