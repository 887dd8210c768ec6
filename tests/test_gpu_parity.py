"""GPU parity: every entry point of the C ABI against the fp64 oracle.

Small seeded cases that span several 32-key / 16-row tiles with ragged tails,
each split plan, both head dimensions, both storage types, the edge cases, and
the first two workloads end to end (the fp32 tiny head and the Qwen3-4B-shaped
decode layer at full size).
"""
import numpy as np
import pytest

import oracle
from helpers import (ATOL_F32, ATOL_LSE_BF16, ATOL_OUT_BF16, REL_L2_BF16, check, dev, host)
from learned_kv_cache_02_amd import configs, synth

pytestmark = pytest.mark.gpu

ACTS = {"gelu": 0, "silu": 1, "gelu_tanh": 2}    # nectar_act values


@pytest.fixture(scope="module")
def nx(gpu):
    from learned_kv_cache_02_amd import nectar
    return nectar


def _bf(x):
    return synth.to_bf16_bits(x)


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence([7919] + list(key)))


def _store(x, dt):
    return _bf(x) if dt == "bf16" else x.astype(np.float32)


# --- exact document attention ---------------------------------------------------

@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("R,Hq,Hkv,n", [(1, 32, 8, 1000), (3, 28, 4, 777), (20, 8, 2, 96), (2, 4, 4, 33),
                                        (10, 16, 4, 500), (70, 16, 4, 1000), (64, 32, 8, 3000)])
@pytest.mark.parametrize("splits", [0, 1, 7])
def test_doc_attn_bf16(nx, d, R, Hq, Hkv, n, splits):
    print("case doc_attn bf16 d=%d R=%d Hq=%d Hkv=%d n=%d splits=%d" % (d, R, Hq, Hkv, n, splits), flush=True)
    g = _rng(1, d, R, Hq, Hkv, n)
    q, K, V = (_bf(g.standard_normal(s)) for s in ((R, Hq, d), (Hkv, n, d), (Hkv, n, d)))
    a, A = nx.doc_attn_exact(dev(q), dev(K), dev(V), Hkv, splits=splits)
    ea, eA = oracle.doc_attn(q, K, V, dt="bf16", Hq=Hq, Hkv=Hkv)
    check("alpha", host(a), ea, 1e-3)
    check("A", host(A), eA, ATOL_OUT_BF16, REL_L2_BF16)


@pytest.mark.parametrize("d,R,n,splits", [(128, 300, 700, 7), (128, 300, 700, 0), (64, 520, 300, 5)])
def test_doc_attn_many_rows(nx, d, R, n, splits):
    """Over 8,192 rows (d = 128) or 16,384 rows (d = 64): the split-K combine
    runs one wave per row over all dims instead of 16-dim row slices."""
    Hq, Hkv = 32, 8
    print("case doc_attn many rows d=%d R=%d n=%d splits=%d" % (d, R, n, splits), flush=True)
    g = _rng(30, d, R, n, splits)
    q, K, V = (_bf(g.standard_normal(s)) for s in ((R, Hq, d), (Hkv, n, d), (Hkv, n, d)))
    a, A = nx.doc_attn_exact(dev(q), dev(K), dev(V), Hkv, splits=splits)
    ea, eA = oracle.doc_attn(q, K, V, dt="bf16", Hq=Hq, Hkv=Hkv)
    check("alpha", host(a), ea, 1e-3)
    check("A", host(A), eA, ATOL_OUT_BF16, REL_L2_BF16)


@pytest.mark.parametrize("n", [19217, 61457])
def test_doc_attn_balanced_splits(nx, n):
    """Decode rows (4 per KV head): the automatic plan spreads the 64-key batches
    over 256 splits per head unevenly (301 batches: one or two per split; 961:
    three or four) with a ragged last batch."""
    R, Hq, Hkv, d = 1, 32, 8, 128
    print("case doc_attn balanced splits n=%d" % n, flush=True)
    g = _rng(3, n)
    q, K, V = (_bf(g.standard_normal(s)) for s in ((R, Hq, d), (Hkv, n, d), (Hkv, n, d)))
    a, A = nx.doc_attn_exact(dev(q), dev(K), dev(V), Hkv)
    ea, eA = oracle.doc_attn(q, K, V, dt="bf16", Hq=Hq, Hkv=Hkv)
    check("alpha", host(a), ea, 1e-3)
    check("A", host(A), eA, ATOL_OUT_BF16, REL_L2_BF16)
    # the two-pass form follows the same plan and agrees bit for bit
    part = nx.doc_attn_partials(dev(q), dev(K), dev(V), Hkv)
    a2, A2 = nx.doc_attn_combine(part, R, Hq, Hkv, d, n, nx.BF16)
    assert np.array_equal(host(a2), host(a)) and np.array_equal(host(A2), host(A))


def _kv_views(K, V, gap=0):
    """Device views k = kv[:, :, 0], v = kv[:, :, 1 + gap] of one contiguous
    [Hkv][n][2 + gap][d] array holding K and V interleaved by key."""
    Hkv, n, d = K.shape
    kv = np.zeros((Hkv, n, 2 + gap, d), K.dtype)
    kv[:, :, 0], kv[:, :, 1 + gap] = K, V
    t = dev(kv)
    return t[:, :, 0], t[:, :, 1 + gap]


@pytest.mark.parametrize("dt,d,R,Hq,Hkv,n,gap", [("bf16", 128, 1, 32, 8, 3000, 0),      # register-direct
                                                 ("bf16", 128, 1, 32, 8, 20011, 0),     # long document, 4 rows: LDS-staged
                                                 ("bf16", 128, 2, 28, 4, 16384, 1),     # ... 14 rows at the key threshold, stride 3d
                                                 ("bf16", 128, 8, 28, 4, 5000, 0),      # LDS-staged, 56 rows
                                                 ("bf16", 128, 64, 32, 8, 2000, 0),     # 32-row waves, 256 rows
                                                 ("bf16", 128, 8, 28, 4, 1001, 2),      # row stride 4d
                                                 ("bf16", 64, 3, 8, 2, 777, 0),
                                                 ("f32", 128, 5, 6, 2, 300, 0), ("f32", 64, 5, 6, 2, 300, 1)])
def test_doc_attn_interleaved_kv(nx, dt, d, R, Hq, Hkv, n, gap):
    """The document cache as one array with K and V interleaved by key (row
    stride (2 + gap) d): the same kernels over strided rows give the dense
    layout's results bit for bit, for the one-call and two-pass forms."""
    print("case doc_attn interleaved %s d=%d R=%d Hq=%d Hkv=%d n=%d gap=%d" % (dt, d, R, Hq, Hkv, n, gap), flush=True)
    g = _rng(41, d, R, n, gap)
    if dt == "bf16":
        q, K, V = (_bf(g.standard_normal(s)) for s in ((R, Hq, d), (Hkv, n, d), (Hkv, n, d)))
    else:
        q, K, V = (g.standard_normal(s).astype(np.float32) for s in ((R, Hq, d), (Hkv, n, d), (Hkv, n, d)))
    k, v = _kv_views(K, V, gap)
    assert not k.is_contiguous() and k.stride(1) == (2 + gap) * d
    a, A = nx.doc_attn_exact(dev(q), k, v, Hkv)
    a0, A0 = nx.doc_attn_exact(dev(q), dev(K), dev(V), Hkv)
    assert np.array_equal(host(a), host(a0)) and np.array_equal(host(A), host(A0))
    ea, eA = oracle.doc_attn(q, K, V, dt=dt, Hq=Hq, Hkv=Hkv)
    if dt == "bf16":
        check("alpha", host(a), ea, 1e-3)
        check("A", host(A), eA, ATOL_OUT_BF16, REL_L2_BF16)
    else:
        check("alpha", host(a), ea, ATOL_F32)
        check("A", host(A), eA, ATOL_F32)
    part = nx.doc_attn_partials(dev(q), k, v, Hkv)
    a2, A2 = nx.doc_attn_combine(part, R, Hq, Hkv, d, n, nx.BF16 if dt == "bf16" else nx.F32)
    assert np.array_equal(host(a2), host(a)) and np.array_equal(host(A2), host(A))


@pytest.mark.parametrize("name", ["decode_bf16", "both_rows56", "exact_only", "batch64_bf16"])
def test_layer_step_interleaved_kv(nx, name):
    """nectar_layer_step with the document cache interleaved by key: every output
    equal bit for bit to the dense layout's."""
    dt, d, B, Tq, T, T_cap, qoff, Hq, Hkv, n, mod = STEP_CASES[name]
    print("case layer_step interleaved %s" % name, flush=True)
    g = _rng(42, len(name), B, Tq, T)
    R = B * Tq
    q = _store(g.standard_normal((R, Hq, d)), dt)
    Kl, Vl = (_store(g.standard_normal((B, Hkv, T_cap, d)), dt) for _ in range(2))
    K, V = (_store(g.standard_normal((Hkv, n, d)), dt) for _ in range(2))
    module = None
    if mod is not None:
        module = _mlp_dev(nx, _mlp_np(g, Hkv, d, mod[1], mod[2], dt), nx.GELU)
    kw = dict(B=B, Tq=Tq, T_loc=T, q_offset=qoff, module=module, exact=True, pairs=True)
    k, v = _kv_views(K, V)
    o1 = {key: host(t) for key, t in nx.layer_step(dev(q), dev(Kl), dev(Vl), Hkv, k=k, v=v, **kw).items()}
    o0 = {key: host(t) for key, t in nx.layer_step(dev(q), dev(Kl), dev(Vl), Hkv, k=dev(K), v=dev(V), **kw).items()}
    assert sorted(o1) == sorted(o0)
    for key in o0:
        assert np.array_equal(o1[key], o0[key], equal_nan=True), key


@pytest.mark.parametrize("d", [128, 64])
def test_doc_attn_f32(nx, d):
    R, Hq, Hkv, n = 5, 6, 2, 300
    g = _rng(2, d)
    q, K, V = (g.standard_normal(s).astype(np.float32) for s in ((R, Hq, d), (Hkv, n, d), (Hkv, n, d)))
    a, A = nx.doc_attn_exact(dev(q), dev(K), dev(V), Hkv)
    ea, eA = oracle.doc_attn(q, K, V, dt="f32", Hq=Hq, Hkv=Hkv)
    check("alpha", host(a), ea, ATOL_F32)
    check("A", host(A), eA, ATOL_F32)


def test_doc_attn_split_invariance_and_determinism(nx):
    R, Hq, Hkv, n, d = 2, 16, 4, 5000, 128
    g = _rng(3)
    q, K, V = (dev(_bf(g.standard_normal(s))) for s in ((R, Hq, d), (Hkv, n, d), (Hkv, n, d)))
    res = {S: [host(t) for t in nx.doc_attn_exact(q, K, V, Hkv, splits=S)] for S in (1, 7, 128)}
    # P is rounded to bf16 relative to each split's running max, so read-outs of
    # different split plans differ by that rounding (2^-9 relative), not more.
    for S in (7, 128):
        check("alpha S=1 vs S=%d" % S, res[S][0], res[1][0], 1e-5)
        check("A S=1 vs S=%d" % S, res[S][1], res[1][1], 1e-3)
    again = [host(t) for t in nx.doc_attn_exact(q, K, V, Hkv, splits=128)]
    assert np.array_equal(again[0], res[128][0]) and np.array_equal(again[1], res[128][1])


@pytest.mark.parametrize("R,Hq,Hkv,n,splits", [(1, 32, 8, 61440, 0), (3, 28, 4, 777, 0), (64, 32, 8, 3000, 0),
                                              (2, 16, 4, 5000, 1), (1, 8, 2, 0, 0)])
def test_doc_attn_two_pass(nx, R, Hq, Hkv, n, splits):
    """Partials then combine: the oracle's (alpha, A), and bitwise the one-call form
    when that form splits the keys too."""
    print("case doc two-pass R=%d Hq=%d Hkv=%d n=%d splits=%d" % (R, Hq, Hkv, n, splits), flush=True)
    import torch
    d = 128
    g = _rng(12, R, n)
    q, K, V = (_bf(g.standard_normal(s)) for s in ((R, Hq, d), (Hkv, n, d), (Hkv, n, d)))
    qd, Kd, Vd = dev(q), dev(K), dev(V)
    part = nx.doc_attn_partials(qd, Kd, Vd, Hkv, splits=splits)
    a2, A2 = nx.doc_attn_combine(part, R, Hq, Hkv, d, n, nx.BF16, splits=splits)
    a1, A1 = nx.doc_attn_exact(qd, Kd, Vd, Hkv, splits=splits)
    ea, eA = oracle.doc_attn(q, K, V, dt="bf16", Hq=Hq, Hkv=Hkv)
    check("alpha two-pass", host(a2), ea, ATOL_LSE_BF16)
    check("A two-pass", host(A2), eA, ATOL_OUT_BF16, REL_L2_BF16)
    dsc = nx.desc(R, Hq, Hkv, d, nx.BF16, 0.0, splits)
    if nx.doc_attn_workspace_size(dsc, n) > 0:
        assert torch.equal(a1, a2) and torch.equal(A1, A2)


def test_scaled_query_stress(nx):
    # Large scores (peaky attention): the online max must keep exp2 in range.
    R, Hq, Hkv, n, d = 1, 8, 2, 2000, 128
    g = _rng(4)
    q = _bf(8.0 * g.standard_normal((R, Hq, d)))
    K, V = (_bf(g.standard_normal((Hkv, n, d))) for _ in range(2))
    a, A = nx.doc_attn_exact(dev(q), dev(K), dev(V), Hkv)
    ea, eA = oracle.doc_attn(q, K, V, dt="bf16", Hq=Hq, Hkv=Hkv)
    check("alpha (8x query)", host(a), ea, ATOL_LSE_BF16)
    check("A (8x query)", host(A), eA, ATOL_OUT_BF16)


@pytest.mark.parametrize("R", [1, 12, 40])          # register-direct, 16-row and 32-row LDS-staged kernels
@pytest.mark.parametrize("scale", [0.2, -0.0884, -0.35])
def test_doc_attn_explicit_and_negative_scale(nx, R, scale):
    # An explicit score scale of either sign (Eq. (3.1) with s_j = scale q.k_j):
    # the kernels carry a negative scale by the query's sign.
    Hq, Hkv, n, d = 8, 2, 2500, 128
    g = _rng(40 + R)
    q = _bf(g.standard_normal((R, Hq, d)))
    K, V = (_bf(g.standard_normal((Hkv, n, d))) for _ in range(2))
    print("case doc attn scale %g R %d" % (scale, R), flush=True)
    a, A = nx.doc_attn_exact(dev(q), dev(K), dev(V), Hkv, scale=scale)
    ea, eA = oracle.doc_attn(q, K, V, dt="bf16", Hq=Hq, Hkv=Hkv, scale=scale)
    check("alpha (scale %g)" % scale, host(a), ea, ATOL_LSE_BF16)
    check("A (scale %g)" % scale, host(A), eA, ATOL_OUT_BF16)


def test_doc_attn_empty_document(nx):
    import torch
    R, Hq, Hkv, d = 2, 4, 2, 128
    q = dev(_bf(_rng(5).standard_normal((R, Hq, d))))
    empty = torch.empty((Hkv, 0, d), dtype=torch.bfloat16, device="cuda")
    a, A = nx.doc_attn_exact(q, empty, empty, Hkv)
    assert np.all(host(a) == -np.inf) and np.all(host(A) == 0.0)


# --- Quadrature (KV-pair) module ---------------------------------------------------

@pytest.mark.parametrize("p", [1, 100, 10486])
def test_kvpair_module(nx, p):
    R, Hq, Hkv, d = 8, 28, 4, 128
    g = _rng(6, p)
    q = _bf(g.standard_normal((R, Hq, d)))
    W, Z = (_bf(g.standard_normal((Hkv, p, d))) for _ in range(2))
    a, A = nx.module_forward(dev(q), nx.KVPairModule(dev(W), dev(Z)), Hkv)
    ea, eA = oracle.kvpair(q, W, Z, dt="bf16", Hq=Hq, Hkv=Hkv)
    check("a", host(a), ea, 1e-3)
    check("A", host(A), eA, ATOL_OUT_BF16, REL_L2_BF16)


# --- MLP module ------------------------------------------------------------------------

def _mlp_np(g, Hkv, d, Ht, Hs, dt, bias=0.5):
    P = dict(W1=_store(g.standard_normal((Hkv, Ht, d)) * d ** -0.5, dt),
             W2t=_store(g.standard_normal((Hkv, Ht, d)) * max(Ht, 1) ** -0.5, dt),
             Ws=_store(g.standard_normal((Hkv, Hs, d)) * d ** -0.5, dt),
             ws2=_store(g.standard_normal((Hkv, Hs)) * max(Hs, 1) ** -0.5, dt),
             b1=(bias * g.standard_normal((Hkv, Ht))).astype(np.float32),
             b2=(bias * g.standard_normal((Hkv, d))).astype(np.float32),
             bs=(bias * g.standard_normal((Hkv, Hs))).astype(np.float32),
             bs2=(bias * g.standard_normal(Hkv)).astype(np.float32))
    return P


def _mlp_dev(nx, P, act):
    import torch
    def t(x):
        return dev(x) if x.size else torch.empty(x.shape, dtype=torch.bfloat16 if x.dtype == np.uint16
                                                   else torch.float32, device="cuda")
    return nx.MLPModule(t(P["W1"]), t(P["b1"]), t(P["W2t"]), t(P["b2"]), t(P["Ws"]), t(P["bs"]),
                        t(P["ws2"]), t(P["bs2"]), act=act)


def _mlp_oracle(q, P, dt, Hq, Hkv, act):
    return oracle.mlp(q, P["W1"], P["b1"], P["W2t"], P["b2"], P["Ws"], P["bs"], P["ws2"], P["bs2"],
                      dt=dt, Hq=Hq, Hkv=Hkv, act=act)


@pytest.mark.parametrize("d,R,Ht,Hs,splits", [(128, 300, 256, 128, 3), (128, 300, 320, 192, 0), (64, 520, 100, 70, 4)])
def test_mlp_many_rows(nx, d, R, Ht, Hs, splits):
    """Over 8,192 rows (d = 128) or 16,384 rows (d = 64) with several hidden-unit
    splits: the split reduce runs one wave per row over all dims."""
    Hq, Hkv = 32, 8
    print("case mlp many rows d=%d R=%d Ht=%d Hs=%d splits=%d" % (d, R, Ht, Hs, splits), flush=True)
    g = _rng(31, d, R, Ht, Hs, splits)
    q = _bf(g.standard_normal((R, Hq, d)))
    P = _mlp_np(g, Hkv, d, Ht, Hs, "bf16")
    a, A = nx.module_forward(dev(q), _mlp_dev(nx, P, nx.GELU), Hkv, splits=splits)
    ea, eA = _mlp_oracle(q, P, "bf16", Hq, Hkv, "gelu")
    check("a", host(a), ea, ATOL_LSE_BF16)
    check("A", host(A), eA, ATOL_OUT_BF16, REL_L2_BF16)


@pytest.mark.parametrize("R,Hq,Hkv,Ht,Hs", [(5, 14, 2, 100, 70), (1, 32, 8, 256, 96), (20, 8, 2, 64, 33),
                                             (3, 4, 1, 0, 40), (3, 4, 1, 50, 0), (10, 16, 4, 300, 200),
                                             (64, 32, 8, 600, 300), (10, 16, 4, 256, 128), (64, 32, 8, 640, 320),
                                             (20, 8, 2, 0, 64), (16, 16, 4, 1000, 500), (11, 12, 4, 96, 40),
                                             # 33-64 rows per KV head (the paired decode kernel): no target
                                             # net, no score net, one-tile slots and odd widths
                                             (10, 16, 4, 0, 200), (10, 16, 4, 300, 0), (14, 16, 4, 33, 7),
                                             (12, 20, 4, 1000, 90)])
@pytest.mark.parametrize("act", ["gelu", "silu", "gelu_tanh"])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_mlp_bf16(nx, R, Hq, Hkv, Ht, Hs, act, splits):
    d = 128
    print("case mlp bf16 R=%d Hq=%d Hkv=%d Ht=%d Hs=%d %s splits=%d" % (R, Hq, Hkv, Ht, Hs, act, splits),
          flush=True)
    g = _rng(8, R, Hq, Ht, Hs)
    q = _bf(g.standard_normal((R, Hq, d)))
    P = _mlp_np(g, Hkv, d, Ht, Hs, "bf16")
    a, A = nx.module_forward(dev(q), _mlp_dev(nx, P, ACTS[act]), Hkv, splits=splits)
    ea, eA = _mlp_oracle(q, P, "bf16", Hq, Hkv, act)
    check("a", host(a), ea, ATOL_LSE_BF16)
    check("A", host(A), eA, ATOL_OUT_BF16, REL_L2_BF16)


@pytest.mark.parametrize("act", ["gelu", "silu", "gelu_tanh"])
@pytest.mark.parametrize("R,Hq,Hkv,Ht,Hs", [(300, 28, 4, 100, 70), (600, 32, 8, 256, 33), (520, 8, 2, 7680, 0),
                                             (400, 28, 4, 768, 512)])
def test_mlp_batched_prefill_bf16(nx, R, Hq, Hkv, Ht, Hs, act):
    """Row counts large enough for the LDS-staged batched kernel (ragged rows and units)."""
    d = 128
    print("case mlp prefill R=%d Hq=%d Hkv=%d Ht=%d Hs=%d %s" % (R, Hq, Hkv, Ht, Hs, act), flush=True)
    g = _rng(12, R, Hq, Ht, Hs)
    q = _bf(g.standard_normal((R, Hq, d)))
    P = _mlp_np(g, Hkv, d, Ht, Hs, "bf16")
    a, A = nx.module_forward(dev(q), _mlp_dev(nx, P, ACTS[act]), Hkv)
    toks = np.unique(np.concatenate([[0, R - 1], g.choice(R, 40, replace=False)])).astype(np.int32)
    ea, eA = oracle.mlp(q, P["W1"], P["b1"], P["W2t"], P["b2"], P["Ws"], P["bs"], P["ws2"], P["bs2"],
                        dt="bf16", Hq=Hq, Hkv=Hkv, toks=toks, act=act)
    check("a", host(a)[toks], ea, ATOL_LSE_BF16)
    check("A", host(A)[toks], eA, ATOL_OUT_BF16, REL_L2_BF16)


def test_mlp_d64_and_f32(nx):
    R, Hq, Hkv, Ht, Hs = 6, 8, 2, 70, 45
    for dt, d, tol in (("bf16", 64, ATOL_OUT_BF16), ("f32", 64, ATOL_F32), ("f32", 128, ATOL_F32)):
        g = _rng(9, d, len(dt))
        q = _store(g.standard_normal((R, Hq, d)), dt)
        P = _mlp_np(g, Hkv, d, Ht, Hs, dt)
        a, A = nx.module_forward(dev(q), _mlp_dev(nx, P, nx.GELU), Hkv)
        ea, eA = _mlp_oracle(q, P, dt, Hq, Hkv, "gelu")
        check("a %s d=%d" % (dt, d), host(a), ea, tol if dt == "f32" else ATOL_LSE_BF16)
        check("A %s d=%d" % (dt, d), host(A), eA, tol)


# --- local causal attention and the fused merge -------------------------------------------

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,Tq,T_loc,T_cap,q_offset", [(2, 37, 37, 40, 0), (3, 1, 100, 128, 99),
                                                        (1, 1, 513, 513, 512), (2, 5, 20, 20, 10),
                                                        (2, 1, 0, 8, 0), (2, 100, 100, 100, 0),
                                                        (1, 70, 300, 320, 230)])
def test_local_attn(nx, dt, B, Tq, T_loc, T_cap, q_offset):
    Hq, Hkv, d = 12, 4, 128
    print("case local %s B=%d Tq=%d T_loc=%d q_offset=%d" % (dt, B, Tq, T_loc, q_offset), flush=True)
    g = _rng(10, B, Tq, T_loc, len(dt))
    R = B * Tq
    q = _store(g.standard_normal((R, Hq, d)), dt)
    Kl, Vl = (_store(g.standard_normal((B, Hkv, T_cap, d)), dt) for _ in range(2))
    dl = g.standard_normal((R, Hq)).astype(np.float32) + 5.0
    dA = (0.1 * g.standard_normal((R, Hq, d))).astype(np.float32)
    lse, A, out, olse = nx.local_attn_lse(dev(q), dev(Kl), dev(Vl), Hkv, B=B, Tq=Tq, T_loc=T_loc,
                                          q_offset=q_offset, doc_lse=dev(dl), doc_A=dev(dA))
    el, eA = oracle.local_attn(q, np.ascontiguousarray(Kl[:, :, :T_loc]),
                               np.ascontiguousarray(Vl[:, :, :T_loc]), dt=dt, B=B, Tq=Tq, Hq=Hq,
                               Hkv=Hkv, Tloc=T_loc, q_offset=q_offset)
    eo, eol = oracle.merge(dl, dA, el, eA)
    tl, to = (ATOL_F32, ATOL_F32) if dt == "f32" else (1e-3, ATOL_OUT_BF16)
    check("lambda", host(lse), el, tl)
    check("A_local", host(A), eA, to)
    check("merged out", host(out), eo, to if dt == "f32" else ATOL_OUT_BF16)
    check("merged lse", host(olse), eol, tl)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_merge_kernel(nx, out_dtype):
    import torch
    R, Hq, Hkv, d = 7, 8, 2, 128
    g = _rng(11)
    a = g.standard_normal((R, Hq)).astype(np.float32) * 3
    lam = g.standard_normal((R, Hq)).astype(np.float32) * 3
    a[0, 0] = -np.inf; lam[0, 1] = -np.inf; a[1, 2] = lam[1, 2] = -np.inf; a[2, 3] = 80.0; lam[2, 3] = -80.0
    A, Al = (g.standard_normal((R, Hq, d)).astype(np.float32) for _ in range(2))
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out, lse = nx.merge(dev(a), dev(A), dev(lam), dev(Al), Hkv=Hkv, out_dtype=tdt)
    eo, el = oracle.merge(a, A, lam, Al)
    check("merge out", host(out), eo, 1e-5 if out_dtype == "f32" else 1e-2)
    check("merge lse", host(lse), el, 1e-5)
    assert np.all(host(out)[1, 2] == 0.0) and host(lse)[1, 2] == -np.inf


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("K,local", [(1, True), (3, True), (8, True), (5, False), (0, True)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_merge_k_kernel(nx, d, K, local, out_dtype):
    import torch
    print("case merge_k d=%d K=%d local=%s %s" % (d, K, local, out_dtype), flush=True)
    R, Hq, Hkv = 9, 8, 2
    g = _rng(12, d, K, int(local))
    pairs = []
    for k in range(K):
        a = (g.standard_normal((R, Hq)) * 3).astype(np.float32)
        a[0, k % Hq] = -np.inf                       # a pair that drops out of one row
        a[3, :] = 60.0 + k                           # large logits
        pairs.append((a, g.standard_normal((R, Hq, d)).astype(np.float32)))
    lam = (g.standard_normal((R, Hq)) * 3).astype(np.float32) if local else None
    Al = g.standard_normal((R, Hq, d)).astype(np.float32) if local else None
    for a, _ in pairs:                               # row 1, head 2: every logit -inf
        a[1, 2] = -np.inf
    if local:
        lam[1, 2] = -np.inf
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out, lse = nx.merge_k([(dev(a), dev(A)) for a, A in pairs], dev(lam) if local else None,
                          dev(Al) if local else None, Hkv=Hkv, out_dtype=tdt)
    eo, el = oracle.merge_k(pairs, lam, Al)
    check("merge_k out", host(out), eo, 1e-5 if out_dtype == "f32" else 1e-2)
    check("merge_k lse", host(lse), el, 1e-5)
    assert np.all(host(out)[1, 2] == 0.0) and host(lse)[1, 2] == -np.inf


@pytest.mark.parametrize("cuts", [(0, 1000, 2300, 2301, 4000), (0, 4000), (0, 300, 300, 2000, 3333, 3334, 3900,
                                                                           4000)])
def test_merge_k_of_document_chunks_is_full_attention(nx, cuts):
    """A document cut into key ranges: each range's exact pair on the GPU, the
    local pair on the GPU, their K-way merge against full attention in the oracle."""
    import torch
    print("case merge_k chunks %s" % (cuts,), flush=True)
    B, Tq, Hq, Hkv, d, T_loc, T_cap, qoff = 2, 3, 16, 4, 128, 50, 64, 47
    R = B * Tq
    n = cuts[-1]
    g = _rng(13, len(cuts))
    q = _bf(g.standard_normal((R, Hq, d)))
    K, V = (_bf(g.standard_normal((Hkv, n, d))) for _ in range(2))
    Kl, Vl = (_bf(g.standard_normal((B, Hkv, T_cap, d))) for _ in range(2))
    qd, Kd, Vd = dev(q), dev(K), dev(V)
    pairs = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        pairs.append(nx.doc_attn_exact(qd, Kd[:, lo:hi].contiguous(), Vd[:, lo:hi].contiguous(), Hkv))
    lam, Al = nx.local_attn_lse(qd, dev(Kl), dev(Vl), Hkv, B=B, Tq=Tq, T_loc=T_loc, q_offset=qoff)
    out, lse = nx.merge_k(pairs, lam, Al, Hkv=Hkv, out_dtype=torch.bfloat16)
    flse, fout = oracle.full_attn(q, K, V, np.ascontiguousarray(Kl[:, :, :T_loc]),
                                  np.ascontiguousarray(Vl[:, :, :T_loc]), dt="bf16", B=B, Tq=Tq, Hq=Hq,
                                  Hkv=Hkv, Tloc=T_loc, q_offset=qoff)
    check("chunked merge out", host(out), fout, ATOL_OUT_BF16)
    check("chunked merge lse", host(lse), flse, 1e-3)


def test_worked_example_on_gpu(nx):
    """The printed merge example of section 2.2 through the GPU merge kernel."""
    import math
    import torch
    R, Hq, d = 1, 1, 64
    a = np.array([[math.log(9.0)]], np.float32)
    lam = np.array([[math.log(3.0)]], np.float32)
    A = np.full((R, Hq, d), 2.0, np.float32)
    Al = np.full((R, Hq, d), 10.0, np.float32)
    out, lse = nx.merge(dev(a), dev(A), dev(lam), dev(Al), Hkv=1, out_dtype=torch.float32)
    assert np.allclose(host(out), 4.0, atol=1e-6) and abs(host(lse)[0, 0] - math.log(12.0)) < 1e-6


# --- the fused layer step ----------------------------------------------------------------

STEP_CASES = {
    # name: (dt, d, B, Tq, T_loc, T_cap, q_offset, Hq, Hkv, n, module)
    "decode_bf16": ("bf16", 128, 1, 1, 513, 513, 512, 32, 8, 3000, ("mlp", 256, 96)),
    "batch64_bf16": ("bf16", 128, 64, 1, 300, 320, 299, 32, 8, 2000, ("mlp", 600, 300)),
    "prefill_bf16": ("bf16", 128, 2, 100, 100, 100, 0, 28, 4, 1500, ("mlp", 300, 200)),
    "kvpair_bf16": ("bf16", 128, 8, 1, 257, 384, 256, 28, 4, 5000, ("kvpair", 700)),
    # the pairs' and the local part's LDS-staged blocks in one launch: one partial local
    # stage (40 keys) beside pairs of a ragged last stage (301 = 3 x 96 + 13)
    "kvpair_short_local": ("bf16", 128, 8, 1, 40, 48, 39, 28, 4, None, ("kvpair", 301)),
    # ... a local part of several stages per split (12 x 4 problems, 500 keys: two splits
    # of three stages), and one beyond the paired plan (20 x 4 problems in two splits:
    # more than 128 local blocks, so the pairs and the local pass launch apart)
    "kvpair_local_stages": ("bf16", 128, 12, 1, 500, 512, 499, 28, 4, None, ("kvpair", 1000)),
    "kvpair_many_local": ("bf16", 128, 20, 1, 500, 512, 499, 28, 4, None, ("kvpair", 1000)),
    "tiny_f32_d64": ("f32", 64, 1, 16, 16, 16, 0, 2, 1, 512, ("mlp", 256, 256)),
    "decode_bf16_d64": ("bf16", 64, 3, 1, 40, 48, 39, 8, 2, 777, ("mlp", 100, 70)),
    "empty_doc_and_local": ("bf16", 128, 2, 1, 0, 8, 0, 8, 2, 0, ("mlp", 0, 40)),
    "exact_only": ("bf16", 128, 4, 1, 50, 64, 49, 16, 4, 1000, None),
    "module_only": ("bf16", 128, 4, 2, 30, 32, 28, 16, 4, None, ("mlp", 64, 32)),
    # 56 document rows per KV head (the 1M-token decode's shape): the Nectar path fuses
    # the 64-row module blocks with the local blocks; with the exact part the LDS-staged
    # document pass and the module defer their partials to the same finishing pass
    "nectar_rows56": ("bf16", 128, 8, 1, 300, 320, 299, 28, 4, None, ("mlp", 704, 450)),
    "both_rows56": ("bf16", 128, 8, 1, 300, 320, 299, 28, 4, 3000, ("mlp", 704, 450)),
}


@pytest.mark.parametrize("name", sorted(STEP_CASES))
def test_layer_step(nx, name):
    """nectar_layer_step against the oracle: every pair it writes and both merged
    outputs; the exact output also against full attention over [document; local]."""
    _check_layer_step(nx, name, 0)


@pytest.mark.parametrize("name,splits", [("decode_bf16", 100), ("batch64_bf16", 70), ("decode_bf16_d64", 90),
                                         ("nectar_rows56", 80), ("both_rows56", 80), ("kvpair_bf16", 40)])
def test_layer_step_many_splits(nx, name, splits):
    """More than 64 key splits per part: the finishing pass and the split-K
    combine fold the splits past the 64 they load up front in a serial tail."""
    _check_layer_step(nx, name, splits)


def _check_layer_step(nx, name, splits):
    dt, d, B, Tq, T, T_cap, qoff, Hq, Hkv, n, mod = STEP_CASES[name]
    print("case layer_step %s splits=%d" % (name, splits), flush=True)
    g = _rng(20, len(name), B, Tq, T)
    R = B * Tq
    q = _store(g.standard_normal((R, Hq, d)), dt)
    Kl, Vl = (_store(g.standard_normal((B, Hkv, T_cap, d)), dt) for _ in range(2))
    Klv, Vlv = (np.ascontiguousarray(x[:, :, :T]) for x in (Kl, Vl))
    kw = dict(dt=dt, Hq=Hq, Hkv=Hkv)
    lkw = dict(B=B, Tq=Tq, Tloc=T, q_offset=qoff, **kw)
    exact = n is not None
    k = v = None
    if exact:
        K, V = (_store(g.standard_normal((Hkv, n, d)), dt) for _ in range(2))
        k, v = dev(K), dev(V)
    module = None
    if mod is not None and mod[0] == "mlp":
        P = _mlp_np(g, Hkv, d, mod[1], mod[2], dt)
        module = _mlp_dev(nx, P, nx.GELU)
    elif mod is not None:
        W, Z = (_store(g.standard_normal((Hkv, mod[1], d)), dt) for _ in range(2))
        module = nx.KVPairModule(dev(W), dev(Z))
    o = nx.layer_step(dev(q), dev(Kl), dev(Vl), Hkv, B=B, Tq=Tq, T_loc=T, q_offset=qoff, k=k, v=v,
                      module=module, exact=exact, pairs=True, splits=splits)
    o = {key: host(t) for key, t in o.items()}
    if dt == "f32":
        to = tl = ATOL_F32
        rel = None
    else:
        to, tl, rel = ATOL_OUT_BF16, ATOL_LSE_BF16, REL_L2_BF16
    el, eAl = oracle.local_attn(q, Klv, Vlv, **lkw)
    check("lambda", o["lam"], el, tl)
    check("A_local", o["Aloc"], eAl, to, rel)
    if exact:
        ea, eA = oracle.doc_attn(q, K, V, **kw)
        check("alpha", o["alpha"], ea, tl)
        check("A", o["A"], eA, to, rel)
        flse, fout = oracle.full_attn(q, K, V, Klv, Vlv, **lkw)
        check("exact out vs full attention", o["out_exact"], fout, to, rel)
        check("exact lse vs full attention", o["lse_exact"], flse, tl)
    if module is not None:
        if mod[0] == "mlp":
            em, eAm = _mlp_oracle(q, P, dt, Hq, Hkv, "gelu")
        else:
            em, eAm = oracle.kvpair(q, W, Z, **kw)
        check("module a", o["a"], em, tl)
        check("module A", o["Am"], eAm, to, rel)
        eo, eol = oracle.merge(em, eAm, el, eAl)
        check("nectar out", o["out_nectar"], eo, to, rel)
        check("nectar lse", o["lse_nectar"], eol, tl)


@pytest.mark.parametrize("name", ["batch64_bf16", "decode_bf16"])
def test_layer_step_output_subsets(nx, name):
    """Requesting only some outputs (here the two merged log-normalisers and the
    exact pair) gives the same values as the full request, on both launch plans."""
    import torch
    dt, d, B, Tq, T, T_cap, qoff, Hq, Hkv, n, mod = STEP_CASES[name]
    print("case layer_step subsets %s" % name, flush=True)
    g = _rng(21, B, Tq, T)
    R = B * Tq
    q = dev(_store(g.standard_normal((R, Hq, d)), dt))
    Kl, Vl = (dev(_store(g.standard_normal((B, Hkv, T_cap, d)), dt)) for _ in range(2))
    k, v = (dev(_store(g.standard_normal((Hkv, n, d)), dt)) for _ in range(2))
    module = _mlp_dev(nx, _mlp_np(g, Hkv, d, mod[1], mod[2], dt), nx.GELU)
    kw = dict(B=B, Tq=Tq, T_loc=T, q_offset=qoff, k=k, v=v, module=module, exact=True)
    full = nx.layer_step(q, Kl, Vl, Hkv, pairs=True, **kw)
    f32 = dict(dtype=torch.float32, device="cuda")
    part = {"lse_exact": torch.empty((R, Hq), **f32), "lse_nectar": torch.empty((R, Hq), **f32),
            "alpha": torch.empty((R, Hq), **f32), "A": torch.empty((R, Hq, d), **f32)}
    from learned_kv_cache_02_amd.nectar import StepOutputs, _lib, _ptr, _stream, _ws_args, desc, LocalDesc, dtype_code
    import ctypes
    dsc = desc(R, Hq, Hkv, d, dtype_code(q))
    loc = LocalDesc(B, Tq, T, T_cap, qoff)
    so = StepOutputs(None, _ptr(part["lse_exact"]), _ptr(part["alpha"]), _ptr(part["A"]), None,
                     _ptr(part["lse_nectar"]), None, None, None, None)
    m = module.struct()
    nbytes = int(_lib.nectar_layer_step_workspace_size(ctypes.byref(dsc), n, ctypes.byref(loc), ctypes.byref(m), 1))
    wp, wn = _ws_args(nbytes, q.device)
    assert _lib.nectar_layer_step(ctypes.byref(dsc), n, ctypes.byref(loc), _ptr(q), _ptr(k), _ptr(v), _ptr(Kl),
                                  _ptr(Vl), ctypes.byref(m), ctypes.byref(so), wp, wn, _stream()) == 0
    for key in part:
        check("subset " + key, host(part[key]), host(full[key]).astype(np.float64), 1e-5)


# --- workloads end to end -----------------------------------------------------------------

def _run_layer(nx, cfg, inputs, step=0):
    """All steps of the hot path for one layer: exact and Nectar document parts,
    the local part, and both merges.  Returns host arrays."""
    q, K, V, Kl, Vl, P = inputs
    Hkv = cfg.Hkv
    alpha, A = nx.doc_attn_exact(q, K, V, Hkv)
    a, Am = nx.module_forward(q, _mlp_dev(nx, P, nx.GELU), Hkv)
    lam, Al, out_x, lse_x = nx.local_attn_lse(q, Kl, Vl, Hkv, B=cfg.B, Tq=cfg.Tq, T_loc=cfg.local_len(step),
                                              q_offset=cfg.q_offset(step), doc_lse=alpha, doc_A=A)
    (out_n, lse_n) = nx.local_attn_lse(q, Kl, Vl, Hkv, B=cfg.B, Tq=cfg.Tq, T_loc=cfg.local_len(step),
                                       q_offset=cfg.q_offset(step), doc_lse=a, doc_A=Am,
                                       want_pair=False)
    return [host(t) for t in (alpha, A, a, Am, lam, Al, out_x, lse_x, out_n, lse_n)]


@pytest.mark.parametrize("cfg", [configs.C1, configs.C2], ids=lambda c: c.name)
def test_workload_layer_end_to_end(nx, cfg):
    print("case workload %s layer 0" % cfg.name, flush=True)
    dt = cfg.dtype
    q = synth.queries(cfg)
    K, V = synth.doc_kv(cfg)
    Kl, Vl = synth.local_kv(cfg)
    P = synth.mlp_params(cfg)
    T = cfg.local_len(0)
    ins = (dev(q), dev(K), dev(V), dev(Kl), dev(Vl), P)
    alpha, A, a, Am, lam, Al, out_x, lse_x, out_n, lse_n = _run_layer(nx, cfg, ins)
    kw = dict(dt=dt, Hq=cfg.Hq, Hkv=cfg.Hkv)
    ea, eA = oracle.doc_attn(q, K, V, **kw)
    em, eAm = _mlp_oracle(q, P, dt, cfg.Hq, cfg.Hkv, "gelu")
    Klv, Vlv = (np.ascontiguousarray(x[:, :, :T]) for x in (Kl, Vl))
    el, eAl = oracle.local_attn(q, Klv, Vlv, B=cfg.B, Tq=cfg.Tq, Tloc=T, q_offset=cfg.q_offset(0), **kw)
    flse, fout = oracle.full_attn(q, K, V, Klv, Vlv, B=cfg.B, Tq=cfg.Tq, Tloc=T, q_offset=cfg.q_offset(0), **kw)
    eon, eln = oracle.merge(em, eAm, el, eAl)
    if dt == "f32":
        to = tl = ATOL_F32
        rel = None
    else:
        to, tl, rel = ATOL_OUT_BF16, ATOL_LSE_BF16, REL_L2_BF16
    check("exact alpha", alpha, ea, tl)
    check("exact A", A, eA, to, rel)
    check("mlp a", a, em, tl)
    check("mlp A", Am, eAm, to, rel)
    check("local lambda", lam, el, tl)
    check("local A", Al, eAl, to, rel)
    # Appendix B identity on the GPU path: exact doc pair merged with the local part
    # equals full attention over the concatenated [document; local] cache.
    check("exact merged vs full attn", out_x, fout, to, rel)
    check("exact merged lse vs full", lse_x, flse, tl)
    check("nectar merged out", out_n, eon, to, rel)
    check("nectar merged lse", lse_n, eln, tl)


def test_c2_layer_step_as_timed(nx):
    """The Qwen3-4B-shaped decode layer at full size (n = 61,440, 513 local keys,
    MLP 4608/2944) through nectar_layer_step exactly as the benchmark calls it:
    both paths in one call with every pair requested (the document's balanced
    splits share the launch with the module's blocks, then one finishing pass),
    then each path alone, the document cache interleaved by key.  Every pair and
    both merged outputs against the oracle."""
    cfg = configs.C2
    print("case c2 layer step as timed", flush=True)
    q = synth.queries(cfg)
    K, V = synth.doc_kv(cfg)
    Kl, Vl = synth.local_kv(cfg)
    P = synth.mlp_params(cfg)
    T, qoff = cfg.local_len(0), cfg.q_offset(0)
    qd, Kld, Vld = dev(q), dev(Kl), dev(Vl)
    Kd, Vd = _kv_views(K, V)          # the document cache interleaved by key, as the benchmark stores it
    mod = _mlp_dev(nx, P, nx.GELU)
    kw = dict(dt="bf16", Hq=cfg.Hq, Hkv=cfg.Hkv)
    Klv, Vlv = (np.ascontiguousarray(x[:, :, :T]) for x in (Kl, Vl))
    ea, eA = oracle.doc_attn(q, K, V, **kw)
    em, eAm = _mlp_oracle(q, P, "bf16", cfg.Hq, cfg.Hkv, "gelu")
    el, eAl = oracle.local_attn(q, Klv, Vlv, B=cfg.B, Tq=cfg.Tq, Tloc=T, q_offset=qoff, **kw)
    flse, fout = oracle.full_attn(q, K, V, Klv, Vlv, B=cfg.B, Tq=cfg.Tq, Tloc=T, q_offset=qoff, **kw)
    eon, eln = oracle.merge(em, eAm, el, eAl)
    to, tl, rel = ATOL_OUT_BF16, ATOL_LSE_BF16, REL_L2_BF16
    skw = dict(B=cfg.B, Tq=cfg.Tq, T_loc=T, q_offset=qoff, pairs=True)
    for name, exact, module in (("both paths", True, mod), ("nectar path", False, mod),
                                ("exact path", True, None)):
        o = nx.layer_step(qd, Kld, Vld, cfg.Hkv, k=Kd if exact else None, v=Vd if exact else None,
                          module=module, exact=exact, **skw)
        o = {key: host(t) for key, t in o.items()}
        check(name + ": lambda", o["lam"], el, tl)
        check(name + ": A_local", o["Aloc"], eAl, to, rel)
        if exact:
            check(name + ": alpha", o["alpha"], ea, tl)
            check(name + ": A", o["A"], eA, to, rel)
            check(name + ": exact out vs full attention", o["out_exact"], fout, to, rel)
            check(name + ": exact lse vs full attention", o["lse_exact"], flse, tl)
        if module is not None:
            check(name + ": module a", o["a"], em, tl)
            check(name + ": module A", o["Am"], eAm, to, rel)
            check(name + ": nectar out", o["out_nectar"], eon, to, rel)
            check(name + ": nectar lse", o["lse_nectar"], eln, tl)
