"""Nectar CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain fp64 reference of the Nectar attention hot path (see ``nectar_oracle.c``
for the definitions and the passages of the Nectar reading notes they follow).
Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the HIP library.

Arrays are numpy: bf16 tensors are passed as their raw ``uint16`` bit patterns,
fp32 as ``float32``, fp64 as ``float64``; biases and merge inputs are
``float64`` (fp32 values widen exactly).  Results are ``float64``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nectar_oracle.c")
_LIB = os.path.join(_HERE, "libnectar_oracle.so")

DT = {"f32": 0, "bf16": 1, "f64": 2}
ACT = {"gelu": 0, "silu": 1, "gelu_tanh": 2}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, OpenMP over rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC",
                               "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_long, ctypes.c_double
        lib.oracle_doc_attn.argtypes = [I, I, I, I, I, L, D, P, P, P, P, I, P, P, I]
        lib.oracle_kvpair.argtypes = [I, I, I, I, I, L, D, P, P, P, P, I, P, P, I]
        lib.oracle_local_attn.argtypes = [I, I, I, I, I, I, I, I, D, P, P, P, P, I, P, P, I]
        lib.oracle_full_attn.argtypes = [I, I, I, I, I, I, L, I, I, D, P, P, P, P, P, P, I, P, P, I]
        lib.oracle_mlp.argtypes = [I, I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, I, P, P, I]
        lib.oracle_deep_mlp.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, I, P, P, I]
        lib.oracle_fit_metrics.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P]
        lib.oracle_act_grad.argtypes = [I, D]
        lib.oracle_act_grad.restype = D
        lib.oracle_mlp_loss_grad.argtypes = [I, I, I, I, I, I, I, I] + [P] * 11 + [D, D] + [P] * 9
        lib.oracle_adamw.argtypes = [L, P, P, P, P, D, D, D, D, D, I, D]
        lib.oracle_adamw.restype = None
        lib.oracle_merge.argtypes = [L, I, P, P, P, P, P, P]
        lib.oracle_merge.restype = None
        lib.oracle_merge_k.argtypes = [L, I, I, P, P, P, P, P, P]
        lib.oracle_merge_k.restype = None
        lib.oracle_gelu.argtypes = [D]
        lib.oracle_gelu.restype = D
        lib.oracle_silu.argtypes = [D]
        lib.oracle_silu.restype = D
        lib.oracle_gelu_tanh.argtypes = [D]
        lib.oracle_gelu_tanh.restype = D
        _lib = lib
    return _lib


_NP = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}


def _arr(x, dt):
    a = np.ascontiguousarray(x)
    if a.dtype != _NP[dt]:
        raise TypeError("expected %s array for dtype %s, got %s" % (_NP[dt], dt, a.dtype))
    return a


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _toks(toks, R):
    if toks is None:
        return None, R
    t = np.ascontiguousarray(toks, dtype=np.int32)
    if t.size and (t.min() < 0 or t.max() >= R):
        raise IndexError("token index out of range")
    return t, int(t.size)


def _scale(scale, d):
    return float(scale) if scale else 1.0 / np.sqrt(d)


def doc_attn(q, K, V, *, dt, Hq, Hkv, scale=0.0, toks=None, threads=0):
    """Eq. (3.1) per token/query head.  q [R][Hq][d], K/V [Hkv][n][d].
    Returns (alpha [ntok][Hq], A [ntok][Hq][d]) in float64."""
    q, K, V = _arr(q, dt), _arr(K, dt), _arr(V, dt)
    d = q.shape[-1]
    R = q.size // (Hq * d)
    n = K.size // (Hkv * d)
    t, nt = _toks(toks, R)
    alpha = np.empty((nt, Hq)); A = np.empty((nt, Hq, d))
    rc = _L().oracle_doc_attn(DT[dt], R, Hq, Hkv, d, n, _scale(scale, d), _p(q), _p(K), _p(V),
                              _p(t), nt, _p(alpha), _p(A), threads)
    if rc:
        raise ValueError("oracle_doc_attn failed (%d)" % rc)
    return alpha, A


def kvpair(q, W, Z, *, dt, Hq, Hkv, scale=0.0, toks=None, threads=0):
    """Quadrature module: exact attention over the p pairs (W, Z)."""
    q, W, Z = _arr(q, dt), _arr(W, dt), _arr(Z, dt)
    d = q.shape[-1]
    R = q.size // (Hq * d)
    p = W.size // (Hkv * d)
    t, nt = _toks(toks, R)
    a = np.empty((nt, Hq)); A = np.empty((nt, Hq, d))
    rc = _L().oracle_kvpair(DT[dt], R, Hq, Hkv, d, p, _scale(scale, d), _p(q), _p(W), _p(Z),
                            _p(t), nt, _p(a), _p(A), threads)
    if rc:
        raise ValueError("oracle_kvpair failed (%d)" % rc)
    return a, A


def local_attn(q, Kl, Vl, *, dt, B, Tq, Hq, Hkv, Tloc, q_offset, scale=0.0, toks=None, threads=0):
    """Causal local attention.  q [B*Tq][Hq][d], Kl/Vl [B][Hkv][Tloc][d]."""
    q, Kl, Vl = _arr(q, dt), _arr(Kl, dt), _arr(Vl, dt)
    d = q.shape[-1]
    t, nt = _toks(toks, B * Tq)
    lse = np.empty((nt, Hq)); A = np.empty((nt, Hq, d))
    rc = _L().oracle_local_attn(DT[dt], B, Tq, Hq, Hkv, d, Tloc, q_offset, _scale(scale, d),
                                _p(q), _p(Kl), _p(Vl), _p(t), nt, _p(lse), _p(A), threads)
    if rc:
        raise ValueError("oracle_local_attn failed (%d)" % rc)
    return lse, A


def full_attn(q, K, V, Kl, Vl, *, dt, B, Tq, Hq, Hkv, Tloc, q_offset, scale=0.0, toks=None,
              threads=0):
    """Attention over [document; local] with the causal mask on the local part."""
    q, K, V, Kl, Vl = (_arr(x, dt) for x in (q, K, V, Kl, Vl))
    d = q.shape[-1]
    n = K.size // (Hkv * d)
    t, nt = _toks(toks, B * Tq)
    lse = np.empty((nt, Hq)); out = np.empty((nt, Hq, d))
    rc = _L().oracle_full_attn(DT[dt], B, Tq, Hq, Hkv, d, n, Tloc, q_offset, _scale(scale, d),
                               _p(q), _p(K), _p(V), _p(Kl), _p(Vl), _p(t), nt, _p(lse), _p(out),
                               threads)
    if rc:
        raise ValueError("oracle_full_attn failed (%d)" % rc)
    return lse, out


def mlp(q, W1, b1, W2t, b2, Ws, bs, ws2, bs2, *, dt, Hq, Hkv, act="gelu", toks=None, threads=0):
    """One-hidden-layer score/target MLP module.  Returns (a [ntok][Hq], A [ntok][Hq][d])."""
    q, W1, W2t, Ws, ws2 = (_arr(x, dt) for x in (q, W1, W2t, Ws, ws2))
    b1, b2, bs, bs2 = (_f64(x) for x in (b1, b2, bs, bs2))
    d = q.shape[-1]
    R = q.size // (Hq * d)
    Ht = W1.size // (Hkv * d)
    Hs = Ws.size // (Hkv * d)
    if W2t.size != W1.size or b1.size != Hkv * Ht or b2.size != Hkv * d or bs.size != Hkv * Hs \
            or ws2.size != Hkv * Hs or bs2.size != Hkv:
        raise ValueError("inconsistent MLP parameter shapes")
    t, nt = _toks(toks, R)
    a = np.empty((nt, Hq)); A = np.empty((nt, Hq, d))
    rc = _L().oracle_mlp(DT[dt], R, Hq, Hkv, d, Ht, Hs, ACT[act], _p(W1), _p(b1), _p(W2t), _p(b2),
                         _p(Ws), _p(bs), _p(ws2), _p(bs2), _p(q), _p(t), nt, _p(a), _p(A), threads)
    if rc:
        raise ValueError("oracle_mlp failed (%d)" % rc)
    return a, A


def deep_mlp(q, P, *, dt, Hq, Hkv, act="silu", toks=None, threads=0):
    """Deep MLP module with input re-injection (Eq. (3.6)) and an optional shared
    backbone.  P holds "depth" (D_b, D_s, D_t), "width" (H_b, H_s, H_t), "layers"
    (a list of (Wq, Wh or None, b) in the order backbone, score, target) and the
    read-outs "ws_out", "bs_out", "Wt_out", "bt_out".
    Returns (a [ntok][Hq], A [ntok][Hq][d]) in float64."""
    q = _arr(q, dt)
    d = q.shape[-1]
    R = q.size // (Hq * d)
    depth = np.ascontiguousarray(P["depth"], dtype=np.int32)
    width = np.ascontiguousarray(P["width"], dtype=np.int32)
    layers = P["layers"]
    if len(layers) != int(depth.sum()):
        raise ValueError("deep_mlp: %d layers for depths %s" % (len(layers), tuple(depth)))
    Db, Ds, Dt = (int(x) for x in depth)
    Hb, Hs, Ht = (int(x) for x in width)
    keep = []
    Wq_p, Wh_p, b_p = [], [], []
    for l, (Wq, Wh, b) in enumerate(layers):
        Wq = _arr(Wq, dt); b = _f64(b)
        Wh = _arr(Wh, dt) if Wh is not None else None
        part = 0 if l < Db else (1 if l < Db + Ds else 2)
        first = (0, Db, Db + Ds)[part]
        H = (Hb, Hs, Ht)[part]
        H_in = H if l > first else (Hb if part > 0 and Db > 0 else 0)
        if Wq.size != Hkv * H * d or b.size != Hkv * H or (Wh is None) != (H_in == 0) or \
                (Wh is not None and Wh.size != Hkv * H * H_in):
            raise ValueError("deep_mlp: layer %d has inconsistent shapes" % l)
        keep += [Wq, Wh, b]
        Wq_p.append(Wq.ctypes.data); Wh_p.append(Wh.ctypes.data if Wh is not None else None)
        b_p.append(b.ctypes.data)
    nl = max(len(layers), 1)
    arrs = [(ctypes.c_void_p * nl)(*v) for v in (Wq_p, Wh_p, b_p)]
    ws_out, Wt_out = _arr(P["ws_out"], dt), _arr(P["Wt_out"], dt)
    bs_out, bt_out = _f64(P["bs_out"]), _f64(P["bt_out"])
    Hs_last, Ht_last = (Hs if Ds else Hb), (Ht if Dt else Hb)
    if ws_out.size != Hkv * Hs_last or Wt_out.size != Hkv * d * Ht_last or bs_out.size != Hkv or \
            bt_out.size != Hkv * d:
        raise ValueError("deep_mlp: inconsistent read-out shapes")
    t, nt = _toks(toks, R)
    a = np.empty((nt, Hq)); A = np.empty((nt, Hq, d))
    rc = _L().oracle_deep_mlp(DT[dt], R, Hq, Hkv, d, ACT[act], _p(depth), _p(width), arrs[0], arrs[1],
                              arrs[2], _p(ws_out), _p(bs_out), _p(Wt_out), _p(bt_out), _p(q), _p(t), nt,
                              _p(a), _p(A), threads)
    if rc:
        raise ValueError("oracle_deep_mlp failed (%d)" % rc)
    return a, A


def fit_metrics(q, a, A, alpha, Aex, *, dt, Hq, Hkv):
    """Per-row (score squared error, target squared error, log RTE ratio)
    [R][Hq][3] and their per-KV-head sums [Hkv][3], float64."""
    q = _arr(q, dt)
    d = q.shape[-1]
    R = q.size // (Hq * d)
    a, A, alpha, Aex = (_f64(x) for x in (a, A, alpha, Aex))
    if a.size != R * Hq or alpha.size != R * Hq or A.size != R * Hq * d or Aex.size != R * Hq * d:
        raise ValueError("fit_metrics: inconsistent shapes")
    row = np.empty((R, Hq, 3)); head = np.empty((Hkv, 3))
    with np.errstate(divide="ignore"):
        rc = _L().oracle_fit_metrics(DT[dt], R, Hq, Hkv, d, _p(q), _p(a), _p(A), _p(alpha), _p(Aex), _p(row),
                                     _p(head))
    if rc:
        raise ValueError("oracle_fit_metrics failed (%d)" % rc)
    return row, head


MLP_PARAMS = ("W1", "b1", "W2t", "b2", "Ws", "bs", "ws2", "bs2")


def mlp_loss_grad(q, P, alpha, A_target, *, dt, Hq, Hkv, act="gelu", lam_alpha=0.1, lam_A=1.0):
    """Regression loss (L, L_alpha, L_A) of the one-hidden-layer module P (dict of
    W1, b1, W2t, b2, Ws, bs, ws2, bs2) against the targets, and its gradient
    (dict of float64 arrays with the parameters' shapes)."""
    q = _arr(q, dt)
    d = q.shape[-1]
    R = q.size // (Hq * d)
    W = {k: (_arr(P[k], dt) if k in ("W1", "W2t", "Ws", "ws2") else _f64(P[k])) for k in MLP_PARAMS}
    Ht, Hs = W["W1"].size // (Hkv * d), W["Ws"].size // (Hkv * d)
    alpha, A_target = _f64(alpha), _f64(A_target)
    if alpha.size != R * Hq or A_target.size != R * Hq * d:
        raise ValueError("mlp_loss_grad: inconsistent target shapes")
    g = {k: np.zeros(np.shape(P[k])) for k in MLP_PARAMS}
    loss = np.zeros(3)
    rc = _L().oracle_mlp_loss_grad(DT[dt], R, Hq, Hkv, d, Ht, Hs, ACT[act], *[_p(W[k]) for k in MLP_PARAMS],
                                   _p(q), _p(alpha), _p(A_target), float(lam_alpha), float(lam_A),
                                   *[_p(g[k]) for k in MLP_PARAMS], _p(loss))
    if rc:
        raise ValueError("oracle_mlp_loss_grad failed (%d)" % rc)
    return loss, g


def act_grad(act: str, x: float) -> float:
    return _L().oracle_act_grad(ACT[act], float(x))


def adamw(theta, g, m, v, *, lr, b1=0.9, b2=0.999, eps=1e-8, wd=0.0, step=1, scale=1.0):
    """One AdamW step on float64 copies; returns (theta, m, v)."""
    theta, m, v = (np.array(x, dtype=np.float64, copy=True) for x in (theta, m, v))
    g = _f64(g)
    _L().oracle_adamw(theta.size, _p(theta), _p(g), _p(m), _p(v), lr, b1, b2, eps, wd, int(step), scale)
    return theta, m, v


def merge(a, A, lam, Aloc):
    """Log-sum-exp merge of (a, A) with (lam, A_loc).  Returns (out, lse) in float64."""
    a, A, lam, Aloc = _f64(a), _f64(A), _f64(lam), _f64(Aloc)
    d = A.shape[-1]
    rows = a.size
    if A.size != rows * d or lam.size != rows or Aloc.size != rows * d:
        raise ValueError("inconsistent merge shapes")
    out = np.empty(A.shape); lse = np.empty(a.shape)
    _L().oracle_merge(rows, d, _p(a), _p(A), _p(lam), _p(Aloc), _p(out), _p(lse))
    return out, lse


def merge_k(pairs, lam=None, Aloc=None):
    """K-way merge of document-side pairs [(a_k, A_k)] with the optional local pair
    (lam, Aloc).  Returns (out, lse) in float64."""
    K = len(pairs)
    a = np.ascontiguousarray(np.stack([_f64(p[0]) for p in pairs])) if K else np.zeros((0,))
    A = np.ascontiguousarray(np.stack([_f64(p[1]) for p in pairs])) if K else np.zeros((0,))
    shape_a = _f64(pairs[0][0]).shape if K else _f64(lam).shape
    shape_A = _f64(pairs[0][1]).shape if K else _f64(Aloc).shape
    d = shape_A[-1]
    rows = int(np.prod(shape_a))
    lam_a = _f64(lam) if lam is not None else None
    Aloc_a = _f64(Aloc) if Aloc is not None else None
    for p in pairs:
        if _f64(p[0]).size != rows or _f64(p[1]).size != rows * d:
            raise ValueError("inconsistent merge_k shapes")
    out = np.empty(shape_A); lse = np.empty(shape_a)
    _L().oracle_merge_k(rows, d, K, _p(a) if K else None, _p(A) if K else None, _p(lam_a), _p(Aloc_a),
                        _p(out), _p(lse))
    return out, lse


def gelu(x: float) -> float:
    return _L().oracle_gelu(float(x))


def silu(x: float) -> float:
    return _L().oracle_silu(float(x))


def gelu_tanh(x: float) -> float:
    return _L().oracle_gelu_tanh(float(x))
