"""Entry points captured in a HIP graph and replayed: every replay must give the
eager result bit for bit (every kernel here sums in a fixed order, so the
results are deterministic).  Between replays the outputs are overwritten by
eager work and the stream is synchronized, so a replay that skipped or reused
work would show.  The workspace is sized by an eager call before capture.
"""
import numpy as np
import pytest

from helpers import dev
from learned_kv_cache_02_amd import configs, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nx(gpu):
    from learned_kv_cache_02_amd import nectar
    return nectar


def _replays(torch, run, outs, n=3):
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for k in range(n):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), "replay %d, output %d differs" % (k, i)
    del g


def _bf(g, *s, std=1.0):
    return dev(synth.to_bf16_bits(g.standard_normal(s) * std))


def _mlp(nx, g, Hkv, d, Ht, Hs):
    import torch
    f = lambda *s: dev((0.1 * g.standard_normal(s)).astype(np.float32))
    return nx.MLPModule(_bf(g, Hkv, Ht, d, std=d ** -0.5), f(Hkv, Ht), _bf(g, Hkv, Ht, d, std=Ht ** -0.5), f(Hkv, d),
                        _bf(g, Hkv, Hs, d, std=d ** -0.5), f(Hkv, Hs), _bf(g, Hkv, Hs, std=Hs ** -0.5), f(Hkv))


@pytest.mark.parametrize("name,B,T_loc,T_cap,Hq,Hkv,n,Ht,Hs", [
    ("decode fused", 1, 513, 513, 32, 8, 3000, 256, 96),
    ("batch-64 composed", 64, 300, 320, 32, 8, 2000, 640, 320)])
def test_layer_step_replays(nx, name, B, T_loc, T_cap, Hq, Hkv, n, Ht, Hs):
    import torch
    print("case graph layer step %s" % name, flush=True)
    g = np.random.default_rng(5)
    d = 128
    q = _bf(g, B, Hq, d)
    K, V = _bf(g, Hkv, n, d), _bf(g, Hkv, n, d)
    Kl, Vl = _bf(g, B, Hkv, T_cap, d), _bf(g, B, Hkv, T_cap, d)
    mod = _mlp(nx, g, Hkv, d, Ht, Hs)
    out = nx.layer_step(q, Kl, Vl, Hkv, B=B, Tq=1, T_loc=T_loc, q_offset=T_loc - 1, k=K, v=V, module=mod, pairs=True)
    run = lambda: nx.layer_step(q, Kl, Vl, Hkv, B=B, Tq=1, T_loc=T_loc, q_offset=T_loc - 1, k=K, v=V, module=mod,
                                pairs=True, out=out)
    _replays(torch, run, list(out.values()))


def test_doc_attn_split_and_modules_replays(nx):
    import torch
    print("case graph doc attn, deep module, merge_k, fit metrics", flush=True)
    g = np.random.default_rng(6)
    R, Hq, Hkv, d, n = 150, 56, 8, 128, 5000
    q = _bf(g, R, Hq, d)
    K, V = _bf(g, Hkv, n, d), _bf(g, Hkv, n, d)
    a = torch.empty(R, Hq, device="cuda")
    A = torch.empty(R, Hq, d, device="cuda")
    _replays(torch, lambda: nx.doc_attn_exact(q, K, V, Hkv, splits=7, alpha_out=a, A_out=A), [a, A])
    # the deep module on the batched (LDS-staged) kernel: 1,050 rows per KV head
    P = synth.deep_mlp_params(9, Hkv, d, configs.DeepShape((2, 1, 2), (64, 96, 64)), "bf16", bias_std=0.2)
    t = lambda x: None if x is None else dev(x)
    deep = nx.DeepMLPModule(P["depth"], P["width"], [(t(x), t(y), t(z)) for x, y, z in P["layers"]], t(P["ws_out"]),
                            t(P["bs_out"]), t(P["Wt_out"]), t(P["bt_out"]))
    am, Am = torch.empty_like(a), torch.empty_like(A)
    _replays(torch, lambda: nx.module_forward(q, deep, Hkv, a_out=am, A_out=Am), [am, Am])
    out = torch.empty(R, Hq, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty_like(a)
    pairs = [(a, A), (am, Am)]
    _replays(torch, lambda: nx.merge_k(pairs, Hkv=Hkv, out_dtype=torch.bfloat16, out=out, lse_out=lse), [out, lse])
    row = torch.empty(R, Hq, 3, device="cuda")
    head = torch.empty(Hkv, 3, dtype=torch.float64, device="cuda")
    _replays(torch, lambda: nx.fit_metrics(q, am, Am, a, A, Hkv, row_out=row, head_out=head), [row, head])


def test_training_step_replays_equal_eager_steps(nx):
    """Three eager training steps and three replays of one captured step, from
    the same state, give the same parameters, moments and module arrays."""
    import torch
    print("case graph training step", flush=True)
    g = np.random.default_rng(7)
    R, Hq, Hkv, d, Ht, Hs = 48, 8, 2, 128, 128, 64
    q = _bf(g, R, Hq, d)
    alpha = dev((g.standard_normal((R, Hq)) + 1).astype(np.float32))
    At = dev((0.3 * g.standard_normal((R, Hq, d))).astype(np.float32))
    mod = _mlp(nx, g, Hkv, d, Ht, Hs)
    init = {k: getattr(mod, k).clone() for k in nx.MLP_PARAMS}
    theta0 = nx.mlp_params_flat(mod)
    hp = nx.train_hparams(lr=1e-3, step=1, clip_norm=0.5, weight_decay=0.01)

    def state():
        for k in nx.MLP_PARAMS:
            getattr(mod, k).copy_(init[k])
        return theta0.clone(), torch.zeros_like(theta0), torch.zeros_like(theta0)

    th, m, v = state()
    grad = torch.empty_like(th)
    loss, gn = torch.empty(3, device="cuda"), torch.empty(2, device="cuda")
    for _ in range(3):
        nx.mlp_train_step(q, mod, alpha, At, Hkv, hp, th, m, v, grad=grad, loss=loss, gnorm=gn)
    torch.cuda.synchronize()
    eager = [th.clone(), m.clone(), v.clone()] + [getattr(mod, k).clone() for k in nx.MLP_PARAMS]
    th2, m2, v2 = state()
    th.copy_(th2); m.copy_(m2); v.copy_(v2)
    torch.cuda.synchronize()
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg):
        nx.mlp_train_step(q, mod, alpha, At, Hkv, hp, th, m, v, grad=grad, loss=loss, gnorm=gn)
    # capture runs nothing: restore the state, then replay three steps
    th.copy_(th2); m.copy_(m2); v.copy_(v2)
    state()
    torch.cuda.synchronize()
    for _ in range(3):
        cg.replay()
        torch.cuda.synchronize()
    got = [th, m, v] + [getattr(mod, k) for k in nx.MLP_PARAMS]
    for i, (x, y) in enumerate(zip(got, eager)):
        assert torch.equal(x, y), i
