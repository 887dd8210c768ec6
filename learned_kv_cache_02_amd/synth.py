"""Seeded synthetic inputs for the Nectar hot path (shared by tests and benchmark).

This module holds no arithmetic of the method itself: it only draws the
inputs the method consumes.  The recipe:

* every tensor element is an independent standard normal from numpy's PCG64,
  seeded by ``SeedSequence([config seed, layer, tensor id, head, chunk, step])``
  and drawn in chunks of ``CHUNK`` rows so chunks can be generated in parallel
  without changing the values;
* keys and queries are RoPE'd (the notes' notation, section 2.1, says the cached
  keys and the query are the rotated ones) with the rotate-half convention
  ``theta_i = base ** (-2 i / d)``, angle = position * theta_i, evaluated in
  float64 at absolute positions: document keys at 0..n-1, local token i of a
  question at n + i, a query at its own token's position;
* module weights are scaled to N(0, 1/fan_in) (fan_in = d for the first layer,
  the hidden width for the read-out, d + the state width for a deep layer that
  re-injects the query); biases are zero unless requested;
  Quadrature pairs W, Z are N(0, 1) without RoPE;
* values are rounded float64 -> float32 (round to nearest even) and, for bf16,
  float32 -> bf16 (round to nearest even).  bf16 tensors are returned as their
  raw ``uint16`` bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Config

CHUNK = 16384

# tensor ids in the seed key
T_DOC_K, T_DOC_V, T_LOC_K, T_LOC_V, T_Q = 0, 1, 2, 3, 4
T_MLP = 16          # + 16 * module index + parameter index
T_KVP_W, T_KVP_Z = 8, 9
T_DEEP = 1024      # + 4 * layer + parameter index; read-outs at T_DEEP + 512

_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))
    return _POOL


def normal(key, rows: int, cols: int) -> np.ndarray:
    """[rows][cols] float64 standard normals for one seed key (tuple of ints)."""
    out = np.empty((rows, cols), dtype=np.float64)

    def fill(c):
        lo, hi = c * CHUNK, min(rows, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key) + [c])))
        g.standard_normal(out=out[lo:hi])

    nch = (rows + CHUNK - 1) // CHUNK
    if nch <= 1:
        for c in range(nch):
            fill(c)
    else:
        list(_pool().map(fill, range(nch)))
    return out


def normal_rows(key, lo: int, hi: int, cols: int) -> np.ndarray:
    """Rows [lo, hi) of normal(key, rows, cols); lo must be a multiple of CHUNK."""
    assert lo % CHUNK == 0
    out = np.empty((hi - lo, cols), dtype=np.float64)
    for c in range(lo // CHUNK, (hi + CHUNK - 1) // CHUNK):
        a, b = c * CHUNK, min(hi, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key) + [c])))
        g.standard_normal(out=out[a - lo:b - lo])
    return out


def rope_tables(pos, d: int, base: float):
    """cos/sin [rows][d/2] of the rotate-half RoPE angles pos * base^(-2i/d), float64."""
    half = d // 2
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x: np.ndarray, pos, base: float, tables=None) -> np.ndarray:
    """Rotate-half RoPE of x [rows][d] (float64) at positions pos [rows], float64 math."""
    d = x.shape[-1]
    half = d // 2
    c, s = tables if tables is not None else rope_tables(pos, d, base)
    x1, x2 = x[:, :half], x[:, half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=1)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64/float32 -> float32 (RNE) -> bf16 (RNE) raw bits as uint16."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float64 array to the storage type ("f32" -> float32, "bf16" -> uint16 bits)."""
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of stored values."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def _heads(cfg: Config, layer: int, tid: int, H: int, rows: int, pos=None, scale=1.0,
           extra=()) -> np.ndarray:
    """[H][rows][d] stored tensor; optional RoPE at `pos` and scaling."""
    out = np.empty((H, rows, cfg.d), dtype=np.float32 if cfg.dtype == "f32" else np.uint16)
    tables = rope_tables(pos, cfg.d, cfg.rope_base) if pos is not None else None

    def one(h, lo, hi):
        # rows [lo, hi) of head h; chunk-aligned, so values do not depend on the split
        x = normal_rows((cfg.seed, layer, tid, h) + tuple(extra), lo, hi, cfg.d)
        if tables is not None:
            x = rope(x, None, cfg.rope_base, (tables[0][lo:hi], tables[1][lo:hi]))
        if scale != 1.0:
            x = x * scale
        out[h, lo:hi] = store(x, cfg.dtype)

    jobs = [(h, lo, min(rows, lo + CHUNK)) for h in range(H) for lo in range(0, rows, CHUNK)]
    if len(jobs) <= 1:
        for j in jobs:
            one(*j)
    else:
        list(_pool().map(lambda j: one(*j), jobs))
    return out


def doc_kv(cfg: Config, layer: int = 0, n: int | None = None):
    """Document cache K, V [Hkv][n][d]; K RoPE'd at positions 0..n-1."""
    n = cfg.n if n is None else n
    K = _heads(cfg, layer, T_DOC_K, cfg.Hkv, n, pos=np.arange(n))
    V = _heads(cfg, layer, T_DOC_V, cfg.Hkv, n)
    return K, V


def local_kv(cfg: Config, layer: int = 0):
    """Local caches [B][Hkv][T_cap][d]; K of local token i RoPE'd at n + i."""
    Tc = cfg.T_cap
    K = np.empty((cfg.B, cfg.Hkv, Tc, cfg.d), dtype=np.float32 if cfg.dtype == "f32" else np.uint16)
    V = np.empty_like(K)
    pos = cfg.n + np.arange(Tc)
    for b in range(cfg.B):
        K[b] = _heads(cfg, layer, T_LOC_K, cfg.Hkv, Tc, pos=pos, extra=(b,))
        V[b] = _heads(cfg, layer, T_LOC_V, cfg.Hkv, Tc, extra=(b,))
    return K, V


def queries(cfg: Config, layer: int = 0, step: int = 0) -> np.ndarray:
    """Query tokens of one step, [R][Hq][d], token-major; each RoPE'd at its position."""
    pos = np.asarray(cfg.query_pos(step))
    Tq = cfg.Tq
    q = np.empty((cfg.B, Tq, cfg.Hq, cfg.d), dtype=np.float32 if cfg.dtype == "f32" else np.uint16)
    for b in range(cfg.B):
        x = _heads(cfg, layer, T_Q, cfg.Hq, Tq, pos=pos, extra=(b, step))   # [Hq][Tq][d]
        q[b] = np.transpose(x, (1, 0, 2))
    return q.reshape(cfg.R, cfg.Hq, cfg.d)


def mlp_params(cfg: Config, layer: int = 0, which: int = 0, bias_std: float = 0.0):
    """One-hidden-layer score/target module per KV head.

    Returns dict with W1, W2t [Hkv][Ht][d]; Ws [Hkv][Hs][d]; ws2 [Hkv][Hs] in the
    storage type, and float32 biases b1 [Hkv][Ht], b2 [Hkv][d], bs [Hkv][Hs], bs2 [Hkv].
    W2t[h][j][c] is the weight from hidden unit j to output c.
    """
    m = cfg.mlps[which]
    d, H = cfg.d, cfg.Hkv
    base = T_MLP + 16 * which
    W1 = _heads(cfg, layer, base + 0, H, m.Ht, scale=d ** -0.5)
    W2t = _heads(cfg, layer, base + 2, H, m.Ht, scale=m.Ht ** -0.5)
    Ws = _heads(cfg, layer, base + 4, H, m.Hs, scale=d ** -0.5)
    ws2 = store(normal((cfg.seed, layer, base + 6), H, m.Hs) * m.Hs ** -0.5, cfg.dtype)

    def bias(pid, shape):
        if bias_std == 0.0:
            return np.zeros(shape, dtype=np.float32)
        x = normal((cfg.seed, layer, base + pid), shape[0], int(np.prod(shape[1:])))
        return (x * bias_std).astype(np.float32).reshape(shape)

    return dict(W1=W1, b1=bias(1, (H, m.Ht)), W2t=W2t, b2=bias(3, (H, d)),
                Ws=Ws, bs=bias(5, (H, m.Hs)), ws2=ws2, bs2=bias(7, (H, 1)).reshape(H),
                Ht=m.Ht, Hs=m.Hs)


def kv_pairs(cfg: Config, layer: int = 0, p: int | None = None):
    """Quadrature pairs W, Z [Hkv][p][d] ~ N(0, 1), no RoPE."""
    p = cfg.kv_pairs if p is None else p
    W = _heads(cfg, layer, T_KVP_W, cfg.Hkv, p)
    Z = _heads(cfg, layer, T_KVP_Z, cfg.Hkv, p)
    return W, Z


def deep_mlp_params(seed: int, Hkv: int, d: int, shape, dtype: str, layer: int = 0, bias_std: float = 0.0):
    """Deep module of Eq. (3.6) per KV head (``shape``: configs.DeepShape).

    Returns dict with depth, width, layers [(Wq [Hkv][H][d], Wh [Hkv][H][H_in] or
    None, b [Hkv][H])], ws_out [Hkv][H_s last], bs_out [Hkv], Wt_out [Hkv][d][H_t last],
    bt_out [Hkv][d]; weights in the storage type, biases float32.  A layer that
    reads the query and a state has fan_in d + H_in for both of its matrices."""
    def w(tid, rows, cols, fan_in):
        x = np.stack([normal((seed, layer, tid, h), rows, cols) for h in range(Hkv)]) * fan_in ** -0.5
        return store(x, dtype)

    def bias(tid, shape_):
        if bias_std == 0.0:
            return np.zeros(shape_, dtype=np.float32)
        x = np.stack([normal((seed, layer, tid, h), 1, int(np.prod(shape_[1:])))[0] for h in range(Hkv)])
        return (x * bias_std).astype(np.float32).reshape(shape_)

    layers = []
    for l, (H, H_in) in enumerate(shape.layers()):
        t = T_DEEP + 4 * l
        fan = d + H_in
        layers.append((w(t, H, d, fan), w(t + 1, H, H_in, fan) if H_in else None, bias(t + 2, (Hkv, H))))
    Hs, Ht = shape.last_width(1), shape.last_width(2)
    t = T_DEEP + 512
    return dict(depth=tuple(shape.depth), width=tuple(shape.width), layers=layers,
                ws_out=w(t, 1, Hs, Hs).reshape(Hkv, Hs), bs_out=bias(t + 1, (Hkv,)).reshape(Hkv),
                Wt_out=w(t + 2, d, Ht, Ht), bt_out=bias(t + 3, (Hkv, d)))
