"""Thin ctypes binding of libnectar.so (the C ABI in include/nectar.h).

Argument marshalling only: every step of the path runs in the HIP library.
Tensors are torch tensors on the GPU (contiguous); bf16 inputs may also be
given as uint16 tensors holding bf16 bit patterns.  Calls are asynchronous on
torch's current stream.  A missing library raises at import.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# NECTAR_LIBRARY may name another build of the same library (e.g. a variant
# compiled with different flags); default: the in-tree build.
LIB_PATH = os.environ.get("NECTAR_LIBRARY", os.path.join(_HERE, "libnectar.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError("libnectar.so is not built (run __graft_entry__.build() or "
                      "python learned_kv_cache_02_amd/build_native.py): no fallback path exists")

_lib = ctypes.CDLL(LIB_PATH)

F32, BF16 = 0, 1
MLP, KVPAIR, DEEP_MLP = 0, 1, 2
DEEP_MAX_LAYERS = 16
GELU, SILU, GELU_TANH = 0, 1, 2
STATUS = {0: "NECTAR_OK", 1: "NECTAR_EINVAL", 2: "NECTAR_EUNSUPPORTED", 3: "NECTAR_EWORKSPACE",
          4: "NECTAR_EHIP"}


class AttnDesc(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("splits", ctypes.c_int32), ("kv_stride", ctypes.c_int32)]


class LocalDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Tq", ctypes.c_int32), ("T_loc", ctypes.c_int32),
                ("T_cap", ctypes.c_int32), ("q_offset", ctypes.c_int32)]


class DeepMLP(ctypes.Structure):
    _fields_ = [("depth", ctypes.c_int32 * 3), ("width", ctypes.c_int32 * 3), ("act", ctypes.c_int32),
                ("Wq", ctypes.c_void_p * DEEP_MAX_LAYERS), ("Wh", ctypes.c_void_p * DEEP_MAX_LAYERS),
                ("b", ctypes.c_void_p * DEEP_MAX_LAYERS),
                ("ws_out", ctypes.c_void_p), ("bs_out", ctypes.c_void_p),
                ("Wt_out", ctypes.c_void_p), ("bt_out", ctypes.c_void_p)]


class Module(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("act", ctypes.c_int32), ("Ht", ctypes.c_int32),
                ("Hs", ctypes.c_int32),
                ("W1", ctypes.c_void_p), ("b1", ctypes.c_void_p),
                ("W2t", ctypes.c_void_p), ("b2", ctypes.c_void_p),
                ("Ws", ctypes.c_void_p), ("bs", ctypes.c_void_p),
                ("ws2", ctypes.c_void_p), ("bs2", ctypes.c_void_p),
                ("p", ctypes.c_int64), ("W", ctypes.c_void_p), ("Z", ctypes.c_void_p),
                ("deep", ctypes.POINTER(DeepMLP))]


class TrainHParams(ctypes.Structure):
    _fields_ = [("lambda_alpha", ctypes.c_float), ("lambda_A", ctypes.c_float), ("lr", ctypes.c_float),
                ("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("clip_norm", ctypes.c_float), ("step", ctypes.c_int32)]


class StepOutputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("out_exact", "lse_exact", "alpha_out", "A_out", "out_nectar",
                                                "lse_nectar", "a_out", "Am_out", "lam_out", "Aloc_out")]


_P = ctypes.c_void_p
_D = ctypes.POINTER(AttnDesc)
_lib.nectar_doc_attn_workspace_size.argtypes = [_D, ctypes.c_int64]
_lib.nectar_doc_attn_workspace_size.restype = ctypes.c_size_t
_lib.nectar_doc_attn_exact.argtypes = [_D, ctypes.c_int64, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.nectar_module_workspace_size.argtypes = [_D, ctypes.POINTER(Module)]
_lib.nectar_module_workspace_size.restype = ctypes.c_size_t
_lib.nectar_module_forward.argtypes = [_D, ctypes.POINTER(Module), _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.nectar_local_workspace_size.argtypes = [_D, ctypes.POINTER(LocalDesc)]
_lib.nectar_local_workspace_size.restype = ctypes.c_size_t
_lib.nectar_local_attn_lse.argtypes = [_D, ctypes.POINTER(LocalDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       _P, ctypes.c_size_t, _P]
_lib.nectar_merge.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P]
_lib.nectar_mlp_param_count.argtypes = [_D, ctypes.POINTER(Module)]
_lib.nectar_mlp_param_count.restype = ctypes.c_int64
_lib.nectar_mlp_train_workspace_size.argtypes = [_D, ctypes.POINTER(Module)]
_lib.nectar_mlp_train_workspace_size.restype = ctypes.c_size_t
_lib.nectar_mlp_loss_grad.argtypes = [_D, ctypes.POINTER(Module), _P, _P, _P, ctypes.c_float, ctypes.c_float, _P, _P,
                                      _P, ctypes.c_size_t, _P]
_lib.nectar_adamw_step.argtypes = [ctypes.c_int64, _P, _P, _P, _P, ctypes.POINTER(TrainHParams), _P]
_lib.nectar_mlp_train_step.argtypes = [_D, ctypes.POINTER(Module), _P, _P, _P, ctypes.POINTER(TrainHParams), _P, _P,
                                       _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.nectar_fit_metrics.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.nectar_fit_metrics_workspace_size.argtypes = [_D]
_lib.nectar_fit_metrics_workspace_size.restype = ctypes.c_size_t
_lib.nectar_merge_k.argtypes = [_D, ctypes.c_int, ctypes.POINTER(_P), ctypes.POINTER(_P), _P, _P, _P, _P, _P]
_lib.nectar_doc_attn_partials_size.argtypes = [_D, ctypes.c_int64]
_lib.nectar_doc_attn_partials_size.restype = ctypes.c_size_t
_lib.nectar_doc_attn_partials.argtypes = [_D, ctypes.c_int64, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.nectar_doc_attn_combine.argtypes = [_D, ctypes.c_int64, _P, ctypes.c_size_t, _P, _P, _P]
_lib.nectar_layer_step_workspace_size.argtypes = [_D, ctypes.c_int64, ctypes.POINTER(LocalDesc),
                                                  ctypes.POINTER(Module), ctypes.c_int]
_lib.nectar_layer_step_workspace_size.restype = ctypes.c_size_t
_lib.nectar_layer_step.argtypes = [_D, ctypes.c_int64, ctypes.POINTER(LocalDesc), _P, _P, _P, _P, _P,
                                   ctypes.POINTER(Module), ctypes.POINTER(StepOutputs), _P, ctypes.c_size_t, _P]
_lib.nectar_layer_step_static.argtypes = [_D, ctypes.c_int64, ctypes.POINTER(LocalDesc), _P, _P, _P, _P, _P,
                                          ctypes.POINTER(Module), ctypes.POINTER(StepOutputs), _P]
_lib.nectar_status_string.argtypes = [ctypes.c_int]
_lib.nectar_status_string.restype = ctypes.c_char_p
_lib.nectar_abi_version.restype = ctypes.c_int
_lib.nectar_workspace_init.argtypes = [_P, ctypes.c_size_t, _P]
_lib.nectar_workspace_init.restype = ctypes.c_int
for _f in ("nectar_doc_attn_exact", "nectar_module_forward", "nectar_local_attn_lse", "nectar_merge",
           "nectar_merge_k", "nectar_fit_metrics", "nectar_mlp_loss_grad", "nectar_adamw_step",
           "nectar_mlp_train_step", "nectar_layer_step", "nectar_layer_step_static", "nectar_doc_attn_partials",
           "nectar_doc_attn_combine"):
    getattr(_lib, _f).restype = ctypes.c_int


class NectarError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(_lib.nectar_status_string(code).decode())
        self.code = code
        self.status = STATUS.get(code, str(code))


def _check(code: int):
    if code != 0:
        raise NectarError(code)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _kv_ptr(t: Optional[torch.Tensor]):
    """Address of a document K or V argument whose layout _doc_kv has checked
    (possibly a strided view)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.bfloat16, torch.uint16, torch.int16):
        return BF16
    raise TypeError("unsupported element type %s" % t.dtype)


_STORAGE = (torch.float32, torch.bfloat16, torch.uint16, torch.int16)
F32T = torch.float32


def _arg(x, name, shape, dtype):
    """Shape and element type of a tensor argument, checked on the host before any
    library call (the C ABI receives bare pointers and cannot see sizes).  `shape`
    entries of None are free; `dtype` is a storage code (F32 / BF16: fp32, or
    bf16 as bfloat16 or 16-bit integer bits) or a torch dtype."""
    if not isinstance(x, torch.Tensor):
        raise ValueError("%s must be a torch tensor, got %s" % (name, type(x).__name__))
    if x.dim() != len(shape) or any(e is not None and int(a) != int(e) for a, e in zip(x.shape, shape)):
        want = "[" + "][".join("*" if e is None else str(int(e)) for e in shape) + "]"
        raise ValueError("%s has shape %s, expected %s" % (name, list(x.shape), want))
    if isinstance(dtype, int):
        if x.dtype not in _STORAGE or dtype_code(x) != dtype:
            raise ValueError("%s has element type %s, expected %s" % (name, x.dtype, "fp32" if dtype == F32 else "bf16"))
    elif x.dtype != dtype:
        raise ValueError("%s has element type %s, expected %s" % (name, x.dtype, dtype))
    return x


def _on_gpu(ref, *named, strided=()):
    """Every given tensor on the GPU device of `ref` and contiguous, except the
    names in `strided` (whose layout the caller has checked) -- after the shape and
    type checks, so those are reported first."""
    dev = ref.device
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("%s must be in GPU device memory, got a tensor on %s" % (name, t.device))
        if t.device != dev:
            raise ValueError("%s is on %s, the call's tensors are on %s" % (name, t.device, dev))
        if name not in strided and not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)


def _doc_kv(k, v, Hkv, d, code, ref):
    """The document cache k, v [Hkv][n][d]: two contiguous arrays, or two views with
    one row stride s (a multiple of 8, at least d) and head stride n * s -- e.g.
    k = kv[:, :, 0] and v = kv[:, :, 1] of one contiguous [Hkv][n][2][d] array (K
    and V interleaved by key).  Shapes, types and strides checked on the host (the
    device by _on_gpu, which lets these two be strided); returns (n, kv_stride for
    the descriptor, 0 when dense)."""
    _arg(k, "k", (Hkv, None, d), code)
    n = k.shape[1]
    _arg(v, "v", (Hkv, n, d), code)
    if k.is_contiguous() and v.is_contiguous():
        return n, 0
    s_ = k.stride(1)
    if (k.stride(2) != 1 or v.stride(2) != 1 or v.stride(1) != s_ or s_ < d or s_ % 8 or s_ > (1 << 20)
            or (Hkv > 1 and (k.stride(0) != n * s_ or v.stride(0) != n * s_))):
        raise ValueError("k and v must be contiguous [Hkv][n][d] arrays or views with one row stride (a multiple "
                         "of 8, at least d) and head stride n * row stride; got strides %s and %s"
                         % (tuple(k.stride()), tuple(v.stride())))
    return n, s_


def _q(q, name="q"):
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("%s must be a [R][Hq][d] tensor" % name)
    _arg(q, name, (None, None, None), F32 if q.dtype == torch.float32 else BF16)
    return q.shape[0], q.shape[1], q.shape[2], dtype_code(q)


def desc(R, Hq, Hkv, d, dtype, scale=0.0, splits=0, kv_stride=0) -> AttnDesc:
    return AttnDesc(int(R), int(Hq), int(Hkv), int(d), int(dtype), float(scale), int(splits), int(kv_stride))


_ws_cache = {}


def workspace(nbytes: int, device=None) -> Optional[torch.Tensor]:
    """A cached scratch buffer of at least nbytes on the device (None for 0).

    One buffer per device, shared by every call of this binding: calls issued on
    different streams must not overlap in time (the caller orders them; the C ABI
    itself takes a workspace per call).  The buffer only grows, and it may not
    grow while a graph is being captured -- graphs captured earlier would keep
    the released buffer's address -- so run the largest call once before
    capturing."""
    if nbytes == 0:
        return None
    dev = torch.device(device or "cuda")
    key = (dev.type, dev.index)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        if buf is not None and torch.cuda.is_current_stream_capturing():
            raise RuntimeError("the binding's workspace would grow (to %d bytes) during graph capture: run the "
                               "largest call once before capturing" % nbytes)
        # workspace contents need no initialisation; zeroed once for reproducible scratch
        buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf


def _ws_args(nbytes, device):
    buf = workspace(nbytes, device)
    return (_ptr(buf), nbytes) if buf is not None else (None, 0)


def doc_attn_workspace_size(dsc: AttnDesc, n: int) -> int:
    return int(_lib.nectar_doc_attn_workspace_size(ctypes.byref(dsc), int(n)))


def doc_attn_exact(q, k, v, Hkv, *, scale=0.0, splits=0, alpha_out=None, A_out=None):
    """Exact document attention (alpha [R][Hq], A [R][Hq][d] fp32); q [R][Hq][d], k/v [Hkv][n][d]."""
    R, Hq, d, code = _q(q)
    n, kvs = _doc_kv(k, v, Hkv, d, code, q)
    if alpha_out is not None:
        _arg(alpha_out, "alpha_out", (R, Hq), F32T)
    if A_out is not None:
        _arg(A_out, "A_out", (R, Hq, d), F32T)
    _on_gpu(q, ("q", q), ("k", k), ("v", v), ("alpha_out", alpha_out), ("A_out", A_out), strided=("k", "v"))
    dsc = desc(R, Hq, Hkv, d, code, scale, splits, kvs)
    if alpha_out is None:
        alpha_out = torch.empty((R, Hq), dtype=torch.float32, device=q.device)
    if A_out is None:
        A_out = torch.empty((R, Hq, d), dtype=torch.float32, device=q.device)
    wp, wn = _ws_args(doc_attn_workspace_size(dsc, n), q.device)
    _check(_lib.nectar_doc_attn_exact(ctypes.byref(dsc), n, _ptr(q), _kv_ptr(k), _kv_ptr(v), _ptr(alpha_out),
                                      _ptr(A_out), wp, wn, _stream()))
    return alpha_out, A_out


def doc_attn_partials_size(dsc: AttnDesc, n: int) -> int:
    return int(_lib.nectar_doc_attn_partials_size(ctypes.byref(dsc), int(n)))


def doc_attn_partials(q, k, v, Hkv, *, scale=0.0, splits=0, partials=None):
    """First pass of the exact document attention: the split-K partials, into a
    uint8 device tensor (allocated when not given).  Returns the tensor."""
    R, Hq, d, code = _q(q)
    n, kvs = _doc_kv(k, v, Hkv, d, code, q)
    if partials is not None:
        _arg(partials, "partials", (None,), torch.uint8)
    _on_gpu(q, ("q", q), ("k", k), ("v", v), ("partials", partials), strided=("k", "v"))
    dsc = desc(R, Hq, Hkv, d, code, scale, splits, kvs)
    nbytes = int(_lib.nectar_doc_attn_partials_size(ctypes.byref(dsc), n))
    if partials is None:
        partials = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check(_lib.nectar_doc_attn_partials(ctypes.byref(dsc), n, _ptr(q), _kv_ptr(k), _kv_ptr(v), _ptr(partials),
                                         partials.numel(), _stream()))
    return partials


def doc_attn_combine(partials, R, Hq, Hkv, d, n, dtype, *, scale=0.0, splits=0, alpha_out=None, A_out=None):
    """Second pass: (alpha [R][Hq], A [R][Hq][d]) from the partials of the same shapes."""
    _arg(partials, "partials", (None,), torch.uint8)
    if alpha_out is not None:
        _arg(alpha_out, "alpha_out", (R, Hq), F32T)
    if A_out is not None:
        _arg(A_out, "A_out", (R, Hq, d), F32T)
    _on_gpu(partials, ("partials", partials), ("alpha_out", alpha_out), ("A_out", A_out))
    dsc = desc(R, Hq, Hkv, d, dtype, scale, splits)
    dev_ = partials.device
    if alpha_out is None:
        alpha_out = torch.empty((R, Hq), dtype=torch.float32, device=dev_)
    if A_out is None:
        A_out = torch.empty((R, Hq, d), dtype=torch.float32, device=dev_)
    _check(_lib.nectar_doc_attn_combine(ctypes.byref(dsc), n, _ptr(partials), partials.numel(), _ptr(alpha_out),
                                        _ptr(A_out), _stream()))
    return alpha_out, A_out


@dataclass
class MLPModule:
    """One-hidden-layer score/target module per KV head (tensors on the GPU)."""
    W1: torch.Tensor
    b1: torch.Tensor
    W2t: torch.Tensor
    b2: torch.Tensor
    Ws: torch.Tensor
    bs: torch.Tensor
    ws2: torch.Tensor
    bs2: torch.Tensor
    act: int = GELU

    def check(self, Hkv: int, d: int, code: int):
        """Shapes and element types against the call's KV heads, head dimension and
        storage type (weights in the storage type, biases fp32)."""
        Ht, Hs = int(self.W1.shape[-2]) if self.W1.dim() == 3 else -1, int(self.Ws.shape[-2]) if self.Ws.dim() == 3 else -1
        _arg(self.W1, "W1", (Hkv, Ht, d), code)
        _arg(self.W2t, "W2t", (Hkv, Ht, d), code)
        _arg(self.Ws, "Ws", (Hkv, Hs, d), code)
        _arg(self.ws2, "ws2", (Hkv, Hs), code)
        _arg(self.b1, "b1", (Hkv, Ht), F32T)
        _arg(self.b2, "b2", (Hkv, d), F32T)
        _arg(self.bs, "bs", (Hkv, Hs), F32T)
        _arg(self.bs2, "bs2", (Hkv,), F32T)
        return [(k, getattr(self, k)) for k in ("W1", "b1", "W2t", "b2", "Ws", "bs", "ws2", "bs2")]

    def struct(self) -> Module:
        m = Module()
        m.kind, m.act = MLP, self.act
        m.Ht, m.Hs = self.W1.shape[-2], self.Ws.shape[-2]
        m.W1, m.b1, m.W2t, m.b2 = (_ptr(t) for t in (self.W1, self.b1, self.W2t, self.b2))
        m.Ws, m.bs, m.ws2, m.bs2 = (_ptr(t) for t in (self.Ws, self.bs, self.ws2, self.bs2))
        return m


@dataclass
class KVPairModule:
    """Quadrature module: W, Z [Hkv][p][d]."""
    W: torch.Tensor
    Z: torch.Tensor

    def check(self, Hkv: int, d: int, code: int):
        _arg(self.W, "W", (Hkv, None, d), code)
        _arg(self.Z, "Z", (Hkv, self.W.shape[1], d), code)
        return [("W", self.W), ("Z", self.Z)]

    def struct(self) -> Module:
        m = Module()
        m.kind = KVPAIR
        m.p = self.W.shape[-2]
        m.W, m.Z = _ptr(self.W), _ptr(self.Z)
        return m


@dataclass
class DeepMLPModule:
    """Deep MLP module with query re-injection (Eq. (3.6)): depth (D_b, D_s, D_t),
    width (H_b, H_s, H_t); layers = [(Wq, Wh or None, b)] backbone first, then
    score, then target (Wq [Hkv][H][d], Wh [Hkv][H][H_in], b [Hkv][H] fp32);
    read-outs ws_out [Hkv][H_s last], bs_out [Hkv], Wt_out [Hkv][d][H_t last],
    bt_out [Hkv][d]."""
    depth: tuple
    width: tuple
    layers: list
    ws_out: torch.Tensor
    bs_out: torch.Tensor
    Wt_out: torch.Tensor
    bt_out: torch.Tensor
    act: int = SILU

    def check(self, Hkv: int, d: int, code: int):
        depth = [int(x) for x in self.depth]
        width = [int(x) if depth[i] > 0 else 0 for i, x in enumerate(self.width)]
        if len(self.layers) != sum(depth):
            raise ValueError("deep module: %d layers for depths %s" % (len(self.layers), depth))
        named, l = [], 0
        for part in range(3):
            for j in range(depth[part]):
                Wq, Wh, b = self.layers[l]
                H = width[part]
                H_in = H if j > 0 else (width[0] if part > 0 and depth[0] > 0 else 0)
                _arg(Wq, "layer %d Wq" % l, (Hkv, H, d), code)
                if H_in:
                    _arg(Wh, "layer %d Wh" % l, (Hkv, H, H_in), code)
                elif Wh is not None:
                    raise ValueError("layer %d reads only the query: Wh must be None" % l)
                _arg(b, "layer %d b" % l, (Hkv, H), F32T)
                named += [("layer %d Wq" % l, Wq), ("layer %d Wh" % l, Wh), ("layer %d b" % l, b)]
                l += 1
        Hs = width[1] if depth[1] > 0 else width[0]
        Ht = width[2] if depth[2] > 0 else width[0]
        _arg(self.ws_out, "ws_out", (Hkv, Hs), code)
        _arg(self.bs_out, "bs_out", (Hkv,), F32T)
        _arg(self.Wt_out, "Wt_out", (Hkv, d, Ht), code)
        _arg(self.bt_out, "bt_out", (Hkv, d), F32T)
        return named + [("ws_out", self.ws_out), ("bs_out", self.bs_out), ("Wt_out", self.Wt_out),
                        ("bt_out", self.bt_out)]

    def struct(self) -> Module:
        if len(self.layers) > DEEP_MAX_LAYERS:
            raise ValueError("at most %d layers" % DEEP_MAX_LAYERS)
        dm = DeepMLP()
        dm.depth[:] = [int(x) for x in self.depth]
        dm.width[:] = [int(x) for x in self.width]
        dm.act = self.act
        for l, (Wq, Wh, b) in enumerate(self.layers):
            dm.Wq[l], dm.Wh[l], dm.b[l] = _ptr(Wq), _ptr(Wh), _ptr(b)
        dm.ws_out, dm.bs_out, dm.Wt_out, dm.bt_out = (_ptr(t) for t in (self.ws_out, self.bs_out, self.Wt_out,
                                                                         self.bt_out))
        m = Module()
        m.kind = DEEP_MLP
        m.deep = ctypes.pointer(dm)
        m._deep_keep = dm          # the pointed-to description lives as long as the struct
        return m


def module_workspace_size(dsc: AttnDesc, mod) -> int:
    return int(_lib.nectar_module_workspace_size(ctypes.byref(dsc), ctypes.byref(mod.struct())))


def module_forward(q, module, Hkv, *, scale=0.0, splits=0, a_out=None, A_out=None):
    """(a [R][Hq], A [R][Hq][d]) fp32 of an MLPModule, DeepMLPModule or KVPairModule."""
    R, Hq, d, code = _q(q)
    named = module.check(Hkv, d, code)
    if a_out is not None:
        _arg(a_out, "a_out", (R, Hq), F32T)
    if A_out is not None:
        _arg(A_out, "A_out", (R, Hq, d), F32T)
    _on_gpu(q, ("q", q), ("a_out", a_out), ("A_out", A_out), *named)
    dsc = desc(R, Hq, Hkv, d, code, scale, splits)
    m = module.struct()
    if a_out is None:
        a_out = torch.empty((R, Hq), dtype=torch.float32, device=q.device)
    if A_out is None:
        A_out = torch.empty((R, Hq, d), dtype=torch.float32, device=q.device)
    wp, wn = _ws_args(int(_lib.nectar_module_workspace_size(ctypes.byref(dsc), ctypes.byref(m))), q.device)
    _check(_lib.nectar_module_forward(ctypes.byref(dsc), ctypes.byref(m), _ptr(q), _ptr(a_out),
                                      _ptr(A_out), wp, wn, _stream()))
    return a_out, A_out


def local_workspace_size(dsc: AttnDesc, loc: LocalDesc) -> int:
    return int(_lib.nectar_local_workspace_size(ctypes.byref(dsc), ctypes.byref(loc)))


def local_attn_lse(q, k_loc, v_loc, Hkv, *, B, Tq, T_loc, q_offset, scale=0.0, splits=0,
                   want_pair=True, doc_lse=None, doc_A=None, out=None, out_lse=None,
                   lse_out=None, A_out=None):
    """Causal local attention.  k_loc/v_loc [B][Hkv][T_cap][d].

    Returns (lse, A_local) when want_pair, and additionally (out, out_lse) when a
    document pair (doc_lse, doc_A) is given: the merged output in q's dtype.
    """
    R, Hq, d, code = _q(q)
    _arg(k_loc, "k_loc", (B, Hkv, None, d), code)
    T_cap = k_loc.shape[2]
    _arg(v_loc, "v_loc", (B, Hkv, T_cap, d), code)
    for name, t, shape, dt in (("lse_out", lse_out, (R, Hq), F32T), ("A_out", A_out, (R, Hq, d), F32T),
                               ("doc_lse", doc_lse, (R, Hq), F32T), ("doc_A", doc_A, (R, Hq, d), F32T),
                               ("out", out, (R, Hq, d), code), ("out_lse", out_lse, (R, Hq), F32T)):
        if t is not None:
            _arg(t, name, shape, dt)
    _on_gpu(q, ("q", q), ("k_loc", k_loc), ("v_loc", v_loc), ("lse_out", lse_out), ("A_out", A_out),
            ("doc_lse", doc_lse), ("doc_A", doc_A), ("out", out), ("out_lse", out_lse))
    dsc = desc(R, Hq, Hkv, d, code, scale, splits)
    loc = LocalDesc(int(B), int(Tq), int(T_loc), int(T_cap), int(q_offset))
    if want_pair:
        if lse_out is None:
            lse_out = torch.empty((R, Hq), dtype=torch.float32, device=q.device)
        if A_out is None:
            A_out = torch.empty((R, Hq, d), dtype=torch.float32, device=q.device)
    merge = doc_lse is not None
    if merge:
        if out is None:
            out = torch.empty((R, Hq, d), dtype=q.dtype, device=q.device)
        if out_lse is None:
            out_lse = torch.empty((R, Hq), dtype=torch.float32, device=q.device)
    wp, wn = _ws_args(local_workspace_size(dsc, loc), q.device)
    _check(_lib.nectar_local_attn_lse(ctypes.byref(dsc), ctypes.byref(loc), _ptr(q), _ptr(k_loc), _ptr(v_loc),
                                      _ptr(lse_out), _ptr(A_out), _ptr(doc_lse), _ptr(doc_A), _ptr(out),
                                      _ptr(out_lse), wp, wn, _stream()))
    res = ()
    if want_pair:
        res += (lse_out, A_out)
    if merge:
        res += (out, out_lse)
    return res


def merge(a, A, lam, A_loc, *, Hkv, out_dtype, out=None, lse_out=None):
    """Log-sum-exp merge of (a, A) with (lam, A_loc); out in out_dtype (fp32/bf16)."""
    _arg(A, "A", (None, None, None), F32T)
    R, Hq, d = A.shape
    _arg(a, "a", (R, Hq), F32T)
    _arg(lam, "lam", (R, Hq), F32T)
    _arg(A_loc, "A_loc", (R, Hq, d), F32T)
    if out is not None:
        _arg(out, "out", (R, Hq, d), F32 if out_dtype == torch.float32 else BF16)
    if lse_out is not None:
        _arg(lse_out, "lse_out", (R, Hq), F32T)
    _on_gpu(A, ("a", a), ("A", A), ("lam", lam), ("A_loc", A_loc), ("out", out), ("lse_out", lse_out))
    code = F32 if out_dtype == torch.float32 else BF16
    dsc = desc(R, Hq, Hkv, d, code)
    if out is None:
        out = torch.empty((R, Hq, d), dtype=out_dtype, device=A.device)
    if lse_out is None:
        lse_out = torch.empty((R, Hq), dtype=torch.float32, device=A.device)
    _check(_lib.nectar_merge(ctypes.byref(dsc), _ptr(a), _ptr(A), _ptr(lam), _ptr(A_loc), _ptr(out),
                             _ptr(lse_out), _stream()))
    return out, lse_out


MERGE_K_MAX = 8


def merge_k(pairs, lam=None, A_loc=None, *, Hkv, out_dtype, out=None, lse_out=None):
    """K-way log-sum-exp merge of the document-side pairs [(a_k, A_k)] with the
    optional local pair (lam, A_loc); out in out_dtype (fp32/bf16)."""
    ref = pairs[0][1] if pairs else A_loc
    if ref is None:
        raise ValueError("merge_k needs at least one pair")
    R, Hq, d = ref.shape
    code = F32 if out_dtype == torch.float32 else BF16
    dsc = desc(R, Hq, Hkv, d, code)
    for a, A in pairs:
        if a.shape != (R, Hq) or A.shape != (R, Hq, d) or a.dtype != torch.float32 or A.dtype != torch.float32:
            raise ValueError("merge_k: every pair is ([R][Hq], [R][Hq][d]) float32")
    if (lam is None) != (A_loc is None):
        raise ValueError("merge_k: give both lam and A_loc, or neither")
    if lam is not None:
        _arg(lam, "lam", (R, Hq), F32T)
        _arg(A_loc, "A_loc", (R, Hq, d), F32T)
    if out is not None:
        _arg(out, "out", (R, Hq, d), F32 if out_dtype == torch.float32 else BF16)
    if lse_out is not None:
        _arg(lse_out, "lse_out", (R, Hq), F32T)
    _on_gpu(ref, *[("a[%d]" % i, a) for i, (a, _) in enumerate(pairs)],
            *[("A[%d]" % i, A) for i, (_, A) in enumerate(pairs)], ("lam", lam), ("A_loc", A_loc), ("out", out),
            ("lse_out", lse_out))
    if out is None:
        out = torch.empty((R, Hq, d), dtype=out_dtype, device=ref.device)
    if lse_out is None:
        lse_out = torch.empty((R, Hq), dtype=torch.float32, device=ref.device)
    K = len(pairs)
    pa = (_P * max(K, 1))(*[_ptr(a) for a, _ in pairs])
    pA = (_P * max(K, 1))(*[_ptr(A) for _, A in pairs])
    _check(_lib.nectar_merge_k(ctypes.byref(dsc), K, pa, pA, _ptr(lam), _ptr(A_loc), _ptr(out),
                               _ptr(lse_out), _stream()))
    return out, lse_out


def fit_metrics(q, a, A, alpha, A_exact, Hkv, *, row_out=None, head_out=None):
    """Per row (a - alpha)^2, ||A - A_exact||^2, log(||A - A_exact||^2 / ||q - A_exact||^2)
    ([R][Hq][3] fp32) and their per-KV-head sums ([Hkv][3] fp64)."""
    R, Hq, d, code = _q(q)
    for name, t, shape, dt in (("a", a, (R, Hq), F32T), ("A", A, (R, Hq, d), F32T), ("alpha", alpha, (R, Hq), F32T),
                               ("A_exact", A_exact, (R, Hq, d), F32T), ("row_out", row_out, (R, Hq, 3), F32T),
                               ("head_out", head_out, (Hkv, 3), torch.float64)):
        if t is not None:
            _arg(t, name, shape, dt)
    _on_gpu(q, ("q", q), ("a", a), ("A", A), ("alpha", alpha), ("A_exact", A_exact), ("row_out", row_out),
            ("head_out", head_out))
    dsc = desc(R, Hq, Hkv, d, code)
    if row_out is None:
        row_out = torch.empty((R, Hq, 3), dtype=torch.float32, device=q.device)
    if head_out is None:
        head_out = torch.empty((Hkv, 3), dtype=torch.float64, device=q.device)
    wp, wn = _ws_args(int(_lib.nectar_fit_metrics_workspace_size(ctypes.byref(dsc))), q.device)
    _check(_lib.nectar_fit_metrics(ctypes.byref(dsc), _ptr(q), _ptr(a), _ptr(A), _ptr(alpha), _ptr(A_exact),
                                   _ptr(row_out), _ptr(head_out), wp, wn, _stream()))
    return row_out, head_out


MLP_PARAMS = ("W1", "b1", "W2t", "b2", "Ws", "bs", "ws2", "bs2")


def mlp_params_flat(module: "MLPModule") -> torch.Tensor:
    """The module's parameters as one flat fp32 vector in the training order
    W1, b1, W2t, b2, Ws, bs, ws2, bs2."""
    return torch.cat([getattr(module, k).float().reshape(-1) for k in MLP_PARAMS])


def mlp_grad_split(flat: torch.Tensor, module: "MLPModule") -> dict:
    """Views of a flat vector in the module's parameter shapes."""
    out, o = {}, 0
    for k in MLP_PARAMS:
        t = getattr(module, k)
        out[k] = flat[o:o + t.numel()].view(t.shape)
        o += t.numel()
    return out


def train_hparams(*, lr, step, lambda_alpha=0.1, lambda_A=1.0, beta1=0.9, beta2=0.999, eps=1e-8,
                  weight_decay=0.0, clip_norm=1.0) -> TrainHParams:
    return TrainHParams(lambda_alpha, lambda_A, lr, beta1, beta2, eps, weight_decay, clip_norm, int(step))


def lr_at(step: int, peak: float, warmup: int, total: int) -> float:
    """Warm-up then cosine decay to zero (the notes' schedule, peak 1e-4)."""
    if step <= warmup:
        return peak * step / max(1, warmup)
    t = min(1.0, (step - warmup) / max(1, total - warmup))
    return 0.5 * peak * (1.0 + math.cos(math.pi * t))


def mlp_loss_grad(q, module: "MLPModule", alpha, A_target, Hkv, *, lambda_alpha=0.1, lambda_A=1.0):
    """(grad flat fp32, loss [3] = (L, L_alpha, L_A)) of the regression loss."""
    R, Hq, d, code = _q(q)
    named = module.check(Hkv, d, code)
    _arg(alpha, "alpha", (R, Hq), F32T)
    _arg(A_target, "A_target", (R, Hq, d), F32T)
    _on_gpu(q, ("q", q), ("alpha", alpha), ("A_target", A_target), *named)
    dsc = desc(R, Hq, Hkv, d, code)
    m = module.struct()
    n = int(_lib.nectar_mlp_param_count(ctypes.byref(dsc), ctypes.byref(m)))
    grad = torch.empty(n, dtype=torch.float32, device=q.device)
    loss = torch.empty(3, dtype=torch.float32, device=q.device)
    wp, wn = _ws_args(int(_lib.nectar_mlp_train_workspace_size(ctypes.byref(dsc), ctypes.byref(m))), q.device)
    _check(_lib.nectar_mlp_loss_grad(ctypes.byref(dsc), ctypes.byref(m), _ptr(q), _ptr(alpha), _ptr(A_target),
                                     lambda_alpha, lambda_A, _ptr(grad), _ptr(loss), wp, wn, _stream()))
    return grad, loss


def adamw_step(theta, grad, m, v, hp: TrainHParams):
    _arg(theta, "theta", (None,), F32T)
    for name, t in (("grad", grad), ("m", m), ("v", v)):
        _arg(t, name, (theta.numel(),), F32T)
    _on_gpu(theta, ("theta", theta), ("grad", grad), ("m", m), ("v", v))
    _check(_lib.nectar_adamw_step(theta.numel(), _ptr(theta), _ptr(grad), _ptr(m), _ptr(v), ctypes.byref(hp),
                                  _stream()))


def mlp_train_step(q, module: "MLPModule", alpha, A_target, Hkv, hp: TrainHParams, theta, adam_m, adam_v, *,
                   grad=None, loss=None, gnorm=None):
    """One regression training step; updates theta, the moments and the module's
    arrays in place.  Returns (grad, loss, gnorm)."""
    R, Hq, d, code = _q(q)
    named = module.check(Hkv, d, code)
    _arg(alpha, "alpha", (R, Hq), F32T)
    _arg(A_target, "A_target", (R, Hq, d), F32T)
    dsc = desc(R, Hq, Hkv, d, code)
    m = module.struct()
    nparams = int(_lib.nectar_mlp_param_count(ctypes.byref(dsc), ctypes.byref(m)))
    for name, t in (("theta", theta), ("adam_m", adam_m), ("adam_v", adam_v), ("grad", grad)):
        if t is not None:
            _arg(t, name, (nparams,), F32T)
    if loss is not None:
        _arg(loss, "loss", (3,), F32T)
    if gnorm is not None:
        _arg(gnorm, "gnorm", (2,), F32T)
    _on_gpu(q, ("q", q), ("alpha", alpha), ("A_target", A_target), ("theta", theta), ("adam_m", adam_m),
            ("adam_v", adam_v), ("grad", grad), ("loss", loss), ("gnorm", gnorm), *named)
    f32 = dict(dtype=torch.float32, device=q.device)
    grad = torch.empty(theta.numel(), **f32) if grad is None else grad
    loss = torch.empty(3, **f32) if loss is None else loss
    gnorm = torch.empty(2, **f32) if gnorm is None else gnorm
    wp, wn = _ws_args(int(_lib.nectar_mlp_train_workspace_size(ctypes.byref(dsc), ctypes.byref(m))), q.device)
    _check(_lib.nectar_mlp_train_step(ctypes.byref(dsc), ctypes.byref(m), _ptr(q), _ptr(alpha), _ptr(A_target),
                                      ctypes.byref(hp), _ptr(theta), _ptr(adam_m), _ptr(adam_v), _ptr(grad),
                                      _ptr(loss), _ptr(gnorm), wp, wn, _stream()))
    return grad, loss, gnorm


def layer_step(q, k_loc, v_loc, Hkv, *, B, Tq, T_loc, q_offset, k=None, v=None, module=None,
               exact=True, pairs=False, scale=0.0, splits=0, out=None, no_alloc=False):
    """One fused layer step: exact path over k, v [Hkv][n][d] (when `exact`), Nectar path
    through `module` (when given), both merged with causal local attention over
    k_loc/v_loc [B][Hkv][T_cap][d].  Returns a dict of the outputs: out_exact,
    lse_exact, out_nectar, lse_nectar, and with `pairs` also alpha, A, a, Am, lam, Aloc.
    `out` may supply preallocated tensors under the same keys.  `no_alloc` calls the
    allocation-free entry point (the library's own device scratch, no workspace)."""
    R, Hq, d, code = _q(q)
    _arg(k_loc, "k_loc", (B, Hkv, None, d), code)
    T_cap = k_loc.shape[2]
    _arg(v_loc, "v_loc", (B, Hkv, T_cap, d), code)
    n, kvs = 0, 0
    if exact and k is not None:
        n, kvs = _doc_kv(k, v, Hkv, d, code, q)
    named = module.check(Hkv, d, code) if module is not None else []
    shapes = {"out_exact": ((R, Hq, d), code), "lse_exact": ((R, Hq), F32T), "alpha": ((R, Hq), F32T),
              "A": ((R, Hq, d), F32T), "out_nectar": ((R, Hq, d), code), "lse_nectar": ((R, Hq), F32T),
              "a": ((R, Hq), F32T), "Am": ((R, Hq, d), F32T), "lam": ((R, Hq), F32T), "Aloc": ((R, Hq, d), F32T)}
    for key, t in (out or {}).items():
        if key not in shapes:
            raise ValueError("layer_step: unknown output %r" % key)
        _arg(t, "out[%r]" % key, *shapes[key])
    _on_gpu(q, ("q", q), ("k_loc", k_loc), ("v_loc", v_loc), ("k", k if exact else None), ("v", v if exact else None),
            *named, *[("out[%r]" % key, t) for key, t in (out or {}).items()], strided=("k", "v"))
    dsc = desc(R, Hq, Hkv, d, code, scale, splits, kvs)
    loc = LocalDesc(int(B), int(Tq), int(T_loc), int(T_cap), int(q_offset))
    o = dict(out or {})
    f32 = dict(dtype=torch.float32, device=q.device)

    def want(key, shape, dtype=None):
        if key not in o:
            o[key] = torch.empty(shape, dtype=dtype or torch.float32, device=q.device)

    if exact:
        want("out_exact", (R, Hq, d), q.dtype)
        want("lse_exact", (R, Hq))
        if pairs:
            want("alpha", (R, Hq)); want("A", (R, Hq, d))
    if module is not None:
        want("out_nectar", (R, Hq, d), q.dtype)
        want("lse_nectar", (R, Hq))
        if pairs:
            want("a", (R, Hq)); want("Am", (R, Hq, d))
    if pairs:
        want("lam", (R, Hq)); want("Aloc", (R, Hq, d))
    so = StepOutputs(*(_ptr(o.get(key)) for key in ("out_exact", "lse_exact", "alpha", "A", "out_nectar",
                                                    "lse_nectar", "a", "Am", "lam", "Aloc")))
    m = module.struct() if module is not None else None
    mp = ctypes.byref(m) if m is not None else None
    if no_alloc:
        _check(_lib.nectar_layer_step_static(ctypes.byref(dsc), n, ctypes.byref(loc), _ptr(q),
                                             _kv_ptr(k) if exact else None, _kv_ptr(v) if exact else None, _ptr(k_loc),
                                             _ptr(v_loc), mp, ctypes.byref(so), _stream()))
        return o
    nbytes = int(_lib.nectar_layer_step_workspace_size(ctypes.byref(dsc), n, ctypes.byref(loc), mp, int(exact)))
    wp, wn = _ws_args(nbytes, q.device)
    _check(_lib.nectar_layer_step(ctypes.byref(dsc), n, ctypes.byref(loc), _ptr(q), _kv_ptr(k) if exact else None,
                                  _kv_ptr(v) if exact else None, _ptr(k_loc), _ptr(v_loc), mp, ctypes.byref(so),
                                  wp, wn, _stream()))
    return o


def workspace_init(buf: torch.Tensor):
    """Zero a caller-owned workspace tensor through the library."""
    _on_gpu(buf, ("buf", buf))
    _check(_lib.nectar_workspace_init(_ptr(buf), buf.numel() * buf.element_size(), _stream()))


def abi_version() -> int:
    return int(_lib.nectar_abi_version())
