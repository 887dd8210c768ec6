"""Layer-wise capacity allocation and fit evaluation on the GPU.

* The Qwen2.5-7B-1M-shaped prefill stack with its module capacity allocated by
  layer group as in Table 10 of the Nectar notes (App. C.1: groups [0, 9),
  [9, 15), [15, 27), [27, 28) with multipliers (1, 2, 5, 2), total capacity
  rho = 10 % of 2 n d per layer on average, the score share of the workload's
  7680/5120 module): one layer of each group at its allocated widths (up to
  16,448 / 11,008 hidden units) through the module entry point and the layer
  step at the full 16 x 1,024-token prefill shape, against the oracle on
  sampled tokens.
* A fit evaluation (App. C.4, Eq. (C.1)): regression targets from the exact
  document attention on the GPU, training steps of the module on them, then
  the fit metrics of the trained module on held-out queries.  The trained
  weights are read back and the same evaluation is run in the oracle (exact
  targets, module forward, fit metrics); the GPU pipeline agrees within the
  forward tolerances, and training lowered both errors.
"""
import dataclasses

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


def _allocated():
    cfg = configs.C3
    m = cfg.mlps[1]
    score = m.Hs * (cfg.d + 2) + 1
    return configs.allocated_mlps(cfg, 0.10, score / m.params(cfg.d))


def test_allocation_widths():
    shapes = _allocated()
    assert len(shapes) == 28
    assert len({(s.Ht, s.Hs) for s in shapes}) == 3             # groups 2 and 4 share the multiplier 2
    assert shapes[15].Ht > 9984 and shapes[15].Hs > 6144          # wider than any workload module


@pytest.mark.parametrize("layer", [0, 9, 15, 27])
def test_allocated_stack_layer(nx, layer):
    """One layer of each Table-10 group at its allocated widths."""
    shape = _allocated()[layer]
    cfg = dataclasses.replace(configs.C3, mlps=(shape,))
    print("case allocated layer %d: MLP %d/%d" % (layer, shape.Ht, shape.Hs), flush=True)
    g = np.random.default_rng(layer)
    edge = [0, 1, cfg.Tq - 1, (cfg.B - 1) * cfg.Tq, cfg.R - 1]
    toks = np.unique(np.concatenate([edge, g.choice(cfg.R, 40, replace=False)])).astype(np.int32)
    q = synth.queries(cfg, layer)
    P = synth.mlp_params(cfg, layer)
    Kl, Vl = synth.local_kv(cfg, layer)
    T, qoff = cfg.local_len(0), cfg.q_offset(0)
    kw = dict(dt="bf16", Hq=cfg.Hq, Hkv=cfg.Hkv, toks=toks, threads=16)
    em, eAm = oracle.mlp(q, P["W1"], P["b1"], P["W2t"], P["b2"], P["Ws"], P["bs"], P["ws2"], P["bs2"], **kw)
    Klv, Vlv = (np.ascontiguousarray(x[:, :, :T]) for x in (Kl, Vl))
    el, eAl = oracle.local_attn(q, Klv, Vlv, B=cfg.B, Tq=cfg.Tq, Tloc=T, q_offset=qoff, **kw)
    eo, elo = oracle.merge(em, eAm, el, eAl)
    mod = nx.MLPModule(*(dev(P[k]) for k in ("W1", "b1", "W2t", "b2", "Ws", "bs", "ws2", "bs2")))
    qd = dev(q)
    a, Am = nx.module_forward(qd, mod, cfg.Hkv)
    check("allocated module a", host(a)[toks], em, ATOL_LSE_BF16)
    check("allocated module A", host(Am)[toks], eAm, ATOL_OUT_BF16, REL_L2_BF16)
    o = nx.layer_step(qd, dev(Kl), dev(Vl), cfg.Hkv, B=cfg.B, Tq=cfg.Tq, T_loc=T, q_offset=qoff, module=mod,
                      exact=False, pairs=True)
    check("layer step a", host(o["a"])[toks], em, ATOL_LSE_BF16)
    check("layer step Am", host(o["Am"])[toks], eAm, ATOL_OUT_BF16, REL_L2_BF16)
    check("layer step nectar out", host(o["out_nectar"])[toks], eo, ATOL_OUT_BF16, REL_L2_BF16)
    check("layer step nectar lse", host(o["lse_nectar"])[toks], elo, ATOL_LSE_BF16)


def test_fit_evaluation_after_training(nx):
    """Targets from the exact document attention, training steps, fit metrics of
    the trained module on held-out queries -- the GPU pipeline against the
    oracle's, and the fit better than before training."""
    import torch
    Hkv, Hq, d, n, Ht, Hs = 2, 8, 128, 4096, 256, 128
    R_train, R_eval, steps = 512, 256, 40
    cfg = dataclasses.replace(configs.C2, Hkv=Hkv, Hq=Hq, n=n, B=1, prompt=8, decode_steps=1,
                              mlps=(configs.MLPShape(Ht, Hs),))
    K, V = synth.doc_kv(cfg)
    P = synth.mlp_params(cfg, bias_std=0.1)
    g = np.random.default_rng(np.random.SeedSequence([31, 7]))
    # queries near the keys' scale, so the document pair varies across them
    q_tr = synth.to_bf16_bits(g.standard_normal((R_train, Hq, d)))
    q_ev = synth.to_bf16_bits(g.standard_normal((R_eval, Hq, d)))
    Kd, Vd = dev(K), dev(V)
    mod = nx.MLPModule(*(dev(P[k]) for k in nx.MLP_PARAMS))
    alpha_tr, A_tr = nx.doc_attn_exact(dev(q_tr), Kd, Vd, Hkv)
    alpha_ev, A_ev = nx.doc_attn_exact(dev(q_ev), Kd, Vd, Hkv)

    def evaluate():
        a, Am = nx.module_forward(dev(q_ev), mod, Hkv)
        row, head = nx.fit_metrics(dev(q_ev), a, Am, alpha_ev, A_ev, Hkv)
        return a, Am, host(row), head.cpu().numpy()

    _, _, row0, head0 = evaluate()
    theta = nx.mlp_params_flat(mod)
    m_, v_ = torch.zeros_like(theta), torch.zeros_like(theta)
    qd = dev(q_tr)
    for it in range(1, steps + 1):
        hp = nx.train_hparams(lr=nx.lr_at(it, 3e-3, 5, steps), step=it, clip_norm=1.0)
        nx.mlp_train_step(qd, mod, alpha_tr, A_tr, Hkv, hp, theta, m_, v_)
    a, Am, row1, head1 = evaluate()
    rows = R_eval * Hq
    mse0 = head0.sum(axis=0)[:2] / rows
    mse1 = head1.sum(axis=0)[:2] / rows
    rte0, rte1 = head0[:, 2].sum() / (R_eval * Hq / Hkv), head1[:, 2].sum() / (R_eval * Hq / Hkv)
    print("  score MSE %.4g -> %.4g, target MSE %.4g -> %.4g, RTE term %.3f -> %.3f"
          % (mse0[0], mse1[0], mse0[1], mse1[1], rte0, rte1), flush=True)
    assert mse1[0] < 0.5 * mse0[0] and mse1[1] < mse0[1] and rte1 < rte0

    # the same evaluation in the oracle, from the trained weights read back
    Pt = {k: (host(getattr(mod, k)) if getattr(mod, k).dtype == torch.float32
              else getattr(mod, k).view(torch.int16).cpu().numpy().view(np.uint16)) for k in nx.MLP_PARAMS}
    for k in ("b1", "b2", "bs", "bs2"):
        Pt[k] = Pt[k].astype(np.float32)
    kw = dict(dt="bf16", Hq=Hq, Hkv=Hkv, threads=16)
    ea, eA = oracle.doc_attn(q_ev, K, V, **kw)
    em, eAm = oracle.mlp(q_ev, Pt["W1"], Pt["b1"], Pt["W2t"], Pt["b2"], Pt["Ws"], Pt["bs"], Pt["ws2"], Pt["bs2"], **kw)
    check("targets alpha", host(alpha_ev), ea, ATOL_LSE_BF16)
    check("targets A", host(A_ev), eA, ATOL_OUT_BF16, REL_L2_BF16)
    check("trained module a", host(a), em, ATOL_LSE_BF16)
    check("trained module A", host(Am), eAm, ATOL_OUT_BF16, REL_L2_BF16)
    erow, ehead = oracle.fit_metrics(q_ev, em.astype(np.float32), eAm.astype(np.float32), ea.astype(np.float32),
                                     eA.astype(np.float32), dt="bf16", Hq=Hq, Hkv=Hkv)
    emse = ehead.sum(axis=0)[:2] / rows
    erte = ehead[:, 2].sum() / (R_eval * Hq / Hkv)
    print("  oracle: score MSE %.4g, target MSE %.4g, RTE term %.3f" % (emse[0], emse[1], erte), flush=True)
    # the module outputs agree to ~1e-3 (score) and ~1e-2 relative (read-out), so the
    # layer errors agree to a few percent and the RTE term (a mean of logs) to ~0.05
    assert abs(mse1[0] - emse[0]) <= 0.05 * emse[0] + 1e-4
    assert abs(mse1[1] - emse[1]) <= 0.05 * emse[1]
    assert abs(rte1 - erte) <= 0.05
