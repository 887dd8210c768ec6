"""The allocation-free layer step (nectar_layer_step_static) against the layer
step with a caller workspace (nectar_layer_step): the same plan and kernels on
the same inputs, so the same bits, on consecutive calls of different sizes (the
library's device scratch keeps the previous call's contents); and the oracle on
the smaller call.  The size check runs on the host before any HIP call."""
import ctypes
import os

import numpy as np
import pytest

import oracle
from helpers import ATOL_LSE_BF16, ATOL_OUT_BF16, REL_L2_BF16, check, dev, host
from learned_kv_cache_02_amd import configs, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def nx(gpu):
    from learned_kv_cache_02_amd import nectar
    return nectar


def _inputs(cfg, step=0):
    q = synth.queries(cfg, 0, step)
    K, V = synth.doc_kv(cfg)
    Kl, Vl = synth.local_kv(cfg)
    P = synth.mlp_params(cfg, bias_std=0.3)
    return q, K, V, Kl, Vl, P


def _both(nx, cfg, ins, step=0):
    """The step of both paths with every pair, through both entry points."""
    q, K, V, Kl, Vl, P = ins
    mod = nx.MLPModule(*(dev(P[k]) for k in ("W1", "b1", "W2t", "b2", "Ws", "bs", "ws2", "bs2")))
    kw = dict(B=cfg.B, Tq=cfg.Tq, T_loc=cfg.local_len(step), q_offset=cfg.q_offset(step), k=dev(K), v=dev(V),
              module=mod, exact=True, pairs=True)
    qd, Kld, Vld = dev(q), dev(Kl), dev(Vl)
    ref = {k: host(t) for k, t in nx.layer_step(qd, Kld, Vld, cfg.Hkv, **kw).items()}
    got = {k: host(t) for k, t in nx.layer_step(qd, Kld, Vld, cfg.Hkv, no_alloc=True, **kw).items()}
    assert sorted(ref) == sorted(got)
    for k in ref:
        assert np.array_equal(got[k], ref[k], equal_nan=True), "output %s differs from nectar_layer_step" % k
    return got


def _oracle_check(cfg, ins, o, step=0):
    q, K, V, Kl, Vl, P = ins
    T, qoff = cfg.local_len(step), cfg.q_offset(step)
    kw = dict(dt=cfg.dtype, Hq=cfg.Hq, Hkv=cfg.Hkv)
    Klv, Vlv = (np.ascontiguousarray(x[:, :, :T]) for x in (Kl, Vl))
    el, eAl = oracle.local_attn(q, Klv, Vlv, B=cfg.B, Tq=cfg.Tq, Tloc=T, q_offset=qoff, **kw)
    flse, fout = oracle.full_attn(q, K, V, Klv, Vlv, B=cfg.B, Tq=cfg.Tq, Tloc=T, q_offset=qoff, **kw)
    em, eAm = oracle.mlp(q, P["W1"], P["b1"], P["W2t"], P["b2"], P["Ws"], P["bs"], P["ws2"], P["bs2"], **kw)
    eon, eln = oracle.merge(em, eAm, el, eAl)
    check("exact out vs full attention", o["out_exact"], fout, ATOL_OUT_BF16, REL_L2_BF16)
    check("exact lse vs full attention", o["lse_exact"], flse, ATOL_LSE_BF16)
    check("nectar out", o["out_nectar"], eon, ATOL_OUT_BF16, REL_L2_BF16)
    check("nectar lse", o["lse_nectar"], eln, ATOL_LSE_BF16)


@pytest.mark.gpu
def test_no_alloc_layer_step_two_calls(nx):
    """The 4B decode layer at full size, then a smaller decode layer on the same
    scratch: each bit for bit nectar_layer_step's result."""
    from learned_kv_cache_02_amd.configs import Config, MLPShape
    print("case no-alloc layer step: 4B decode layer, then n = 3,000", flush=True)
    _both(nx, configs.C2, _inputs(configs.C2))
    small = Config("small", 12, "bf16", 1, 4, 16, 128, 3000, 1e6, 2, 40, 1, (MLPShape(320, 192),))
    ins = _inputs(small)
    _oracle_check(small, ins, _both(nx, small, ins))


@pytest.mark.gpu
def test_no_alloc_layer_step_composed_plan(nx):
    """Batch-64 decode rows (256 per KV head): the plan whose parts finish
    themselves (LDS-staged kernels, split combine, in-place merge) on the scratch,
    after a larger call of the same plan."""
    from learned_kv_cache_02_amd.configs import Config, MLPShape
    print("case no-alloc layer step: batch-64 decode, n = 20,000 then 5,000", flush=True)
    for n in (20000, 5000):
        cfg = Config("b64_%d" % n, 13, "bf16", 1, 8, 32, 128, n, 5e5, 64, 40, 4, (MLPShape(640, 384),))
        ins = _inputs(cfg, step=3)
        o = _both(nx, cfg, ins, step=3)
        if n == 5000:
            _oracle_check(cfg, ins, o, step=3)


def test_no_alloc_rejects_oversized_plan_on_host():
    """A plan larger than the scratch (the 16 x 1,024-token prefill's exact path)
    returns NECTAR_EWORKSPACE during validation: fake pointers, nothing launched."""
    from test_abi_cpu import Desc, Local, StepOuts
    lib = ctypes.CDLL(os.path.join(ROOT, "learned_kv_cache_02_amd", "libnectar.so"))
    lib.nectar_layer_step_static.restype = ctypes.c_int
    lib.nectar_layer_step_workspace_size.restype = ctypes.c_size_t
    cfg = configs.C3
    d = Desc(cfg.R, cfg.Hq, cfg.Hkv, cfg.d, 1, 0.0, 0)
    loc = Local(cfg.B, cfg.Tq, cfg.prompt, cfg.prompt, 0)
    fake = ctypes.c_void_p(1 << 20)
    outs = StepOuts(fake, fake, None, None, None, None, None, None, None, None)
    need = lib.nectar_layer_step_workspace_size(ctypes.byref(d), ctypes.c_int64(cfg.n), ctypes.byref(loc), None, 1)
    assert need > (64 << 20)
    st = lib.nectar_layer_step_static(ctypes.byref(d), ctypes.c_int64(cfg.n), ctypes.byref(loc), fake, fake, fake,
                                      fake, fake, None, ctypes.byref(outs), None)
    assert st == 3      # NECTAR_EWORKSPACE
    # an invalid argument is still reported first
    bad = Desc(cfg.R, cfg.Hq, 3, cfg.d, 1, 0.0, 0)
    assert lib.nectar_layer_step_static(ctypes.byref(bad), ctypes.c_int64(cfg.n), ctypes.byref(loc), fake, fake,
                                        fake, fake, fake, None, ctypes.byref(outs), None) == 1
