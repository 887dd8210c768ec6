"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and rejects bad arguments on the host before any HIP call (no GPU needed).

Pointers here are fake addresses; every call below is one the library must
reject during validation, so nothing is ever launched or dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "learned_kv_cache_02_amd", "libnectar.so")
HDR = os.path.join(ROOT, "include", "nectar.h")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = range(5)


class Desc(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("splits", ctypes.c_int32), ("kv_stride", ctypes.c_int32)]


class Local(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Tq", ctypes.c_int32), ("T_loc", ctypes.c_int32),
                ("T_cap", ctypes.c_int32), ("q_offset", ctypes.c_int32)]


DEEP_MAX = 16


class Deep(ctypes.Structure):
    _fields_ = [("depth", ctypes.c_int32 * 3), ("width", ctypes.c_int32 * 3), ("act", ctypes.c_int32),
                ("Wq", ctypes.c_void_p * DEEP_MAX), ("Wh", ctypes.c_void_p * DEEP_MAX),
                ("b", ctypes.c_void_p * DEEP_MAX)] + \
               [(n, ctypes.c_void_p) for n in ("ws_out", "bs_out", "Wt_out", "bt_out")]


class Module(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("act", ctypes.c_int32), ("Ht", ctypes.c_int32),
                ("Hs", ctypes.c_int32)] + \
               [(n, ctypes.c_void_p) for n in ("W1", "b1", "W2t", "b2", "Ws", "bs", "ws2", "bs2")] + \
               [("p", ctypes.c_int64), ("W", ctypes.c_void_p), ("Z", ctypes.c_void_p),
                ("deep", ctypes.POINTER(Deep))]


class HP(ctypes.Structure):
    _fields_ = [(n, ctypes.c_float) for n in ("lambda_alpha", "lambda_A", "lr", "beta1", "beta2", "eps",
                                               "weight_decay", "clip_norm")] + [("step", ctypes.c_int32)]


class StepOuts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("out_exact", "lse_exact", "alpha_out", "A_out", "out_nectar",
                                                "lse_nectar", "a_out", "Am_out", "lam_out", "Aloc_out")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libnectar.so is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    D = ctypes.POINTER(Desc)
    L.nectar_doc_attn_workspace_size.argtypes = [D, ctypes.c_int64]
    L.nectar_doc_attn_workspace_size.restype = ctypes.c_size_t
    L.nectar_doc_attn_exact.argtypes = [D, ctypes.c_int64, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.nectar_module_workspace_size.argtypes = [D, ctypes.POINTER(Module)]
    L.nectar_module_workspace_size.restype = ctypes.c_size_t
    L.nectar_module_forward.argtypes = [D, ctypes.POINTER(Module), P, P, P, P, ctypes.c_size_t, P]
    L.nectar_local_workspace_size.argtypes = [D, ctypes.POINTER(Local)]
    L.nectar_local_workspace_size.restype = ctypes.c_size_t
    L.nectar_local_attn_lse.argtypes = [D, ctypes.POINTER(Local)] + [P] * 9 + [P, ctypes.c_size_t, P]
    L.nectar_merge.argtypes = [D] + [P] * 7
    L.nectar_fit_metrics.argtypes = [D] + [P] * 8 + [ctypes.c_size_t, P]
    L.nectar_fit_metrics_workspace_size.argtypes = [D]
    L.nectar_mlp_param_count.argtypes = [D, ctypes.POINTER(Module)]
    L.nectar_mlp_param_count.restype = ctypes.c_int64
    L.nectar_mlp_train_workspace_size.argtypes = [D, ctypes.POINTER(Module)]
    L.nectar_mlp_train_workspace_size.restype = ctypes.c_size_t
    L.nectar_mlp_loss_grad.argtypes = [D, ctypes.POINTER(Module), P, P, P, ctypes.c_float, ctypes.c_float, P, P, P,
                                       ctypes.c_size_t, P]
    L.nectar_adamw_step.argtypes = [ctypes.c_int64, P, P, P, P, ctypes.POINTER(HP), P]
    L.nectar_mlp_train_step.argtypes = [D, ctypes.POINTER(Module), P, P, P, ctypes.POINTER(HP), P, P, P, P, P, P, P,
                                        ctypes.c_size_t, P]
    L.nectar_fit_metrics_workspace_size.restype = ctypes.c_size_t
    L.nectar_merge_k.argtypes = [D, ctypes.c_int, ctypes.POINTER(P), ctypes.POINTER(P)] + [P] * 5
    L.nectar_layer_step_workspace_size.argtypes = [D, ctypes.c_int64, ctypes.POINTER(Local),
                                                    ctypes.POINTER(Module), ctypes.c_int]
    L.nectar_layer_step_workspace_size.restype = ctypes.c_size_t
    L.nectar_layer_step.argtypes = [D, ctypes.c_int64, ctypes.POINTER(Local), P, P, P, P, P,
                                    ctypes.POINTER(Module), ctypes.POINTER(StepOuts), P, ctypes.c_size_t, P]
    L.nectar_status_string.argtypes = [ctypes.c_int]
    L.nectar_status_string.restype = ctypes.c_char_p
    return L


A16 = 0x10000          # fake, 16-byte aligned
MIS = 0x10004          # fake, only 4-byte aligned


def declared_functions():
    txt = open(HDR).read()
    return sorted(set(re.findall(r"NECTAR_API\s+[\w\s\*]*?\b(nectar_\w+)\s*\(", txt)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 24, names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.nectar_abi_version() == 3


def test_status_strings(lib):
    for code, tag in [(0, b"NECTAR_OK"), (1, b"NECTAR_EINVAL"), (2, b"NECTAR_EUNSUPPORTED"),
                      (3, b"NECTAR_EWORKSPACE"), (4, b"NECTAR_EHIP")]:
        assert lib.nectar_status_string(code).startswith(tag)
    assert b"unknown" in lib.nectar_status_string(99)


def _doc(lib, d, n=64, q=A16, k=A16, v=A16, a=A16, A=A16, ws=A16, wsb=0):
    return lib.nectar_doc_attn_exact(ctypes.byref(d) if d is not None else None, n, q, k, v, a, A,
                                     ws, wsb, None)


def test_doc_attn_validation(lib):
    assert _doc(lib, None) == EINVAL
    assert _doc(lib, Desc(2, 6, 4, 128, 1, 0.0, 0)) == EINVAL            # Hq % Hkv
    assert _doc(lib, Desc(2, 8, 4, 96, 1, 0.0, 0)) == EUNSUPPORTED       # d
    assert _doc(lib, Desc(2, 8, 4, 0, 1, 0.0, 0)) == EINVAL
    assert _doc(lib, Desc(2, 8, 4, 128, 7, 0.0, 0)) == EINVAL            # dtype
    assert _doc(lib, Desc(-1, 8, 4, 128, 1, 0.0, 0)) == EINVAL
    assert _doc(lib, Desc(2, 8, 4, 128, 1, float("nan"), 0)) == EINVAL
    assert _doc(lib, Desc(2, 8, 4, 128, 1, 0.0, -3)) == EINVAL
    # document K/V row stride: 0, or whole 16-byte pieces of at least d elements
    assert _doc(lib, Desc(2, 8, 4, 128, 1, 0.0, 0, 64)) == EINVAL       # shorter than a row
    assert _doc(lib, Desc(2, 8, 4, 128, 1, 0.0, 0, 132)) == EINVAL      # not a multiple of 8
    assert _doc(lib, Desc(2, 8, 4, 128, 1, 0.0, 0, -256)) == EINVAL
    assert _doc(lib, Desc(2, 8, 4, 128, 1, 0.0, 0, 1 << 21)) == EINVAL
    ok = Desc(2, 8, 4, 128, 1, 0.0, 0)
    assert _doc(lib, ok, n=-1) == EINVAL
    assert _doc(lib, ok, q=None) == EINVAL
    assert _doc(lib, ok, q=MIS) == EINVAL                                 # q needs 16 B
    assert _doc(lib, ok, k=None) == EINVAL
    assert _doc(lib, ok, a=A16 + 2) == EINVAL                             # fp32 output alignment
    # A long document needs split partials, so a short workspace is caught
    # before any launch (asserting need > 0 first keeps these calls launch-free).
    need = lib.nectar_doc_attn_workspace_size(ctypes.byref(ok), 100000)
    assert need > 0
    assert _doc(lib, ok, n=100000, ws=A16, wsb=need - 1) == EWORKSPACE
    assert _doc(lib, ok, n=100000, ws=None, wsb=need) == EINVAL
    # R == 0 is a no-op that touches nothing
    assert _doc(lib, Desc(0, 8, 4, 128, 1, 0.0, 0), q=None, k=None, v=None, a=None, A=None) == OK


def test_workspace_sizes(lib):
    # n = 61,440 document keys, 8 KV heads, 4 query heads per group, one token:
    # the entry point's LDS-staged plan, 512 blocks of 32-key stages (two per
    # CU) -> 64 key splits of 30 stages per head, 4 rows per head, (128 + 2)
    # floats per row.  (Forced split counts keep the register-direct plan.)
    d = Desc(1, 32, 8, 128, 1, 0.0, 0)
    assert lib.nectar_doc_attn_workspace_size(ctypes.byref(d), 61440) == 8 * 64 * 4 * 520
    assert lib.nectar_doc_attn_workspace_size(ctypes.byref(d), 0) == 0
    assert lib.nectar_doc_attn_workspace_size(None, 10) == 0
    d1 = Desc(1, 32, 8, 128, 1, 0.0, 1)          # one split: the block finishes rows in place
    assert lib.nectar_doc_attn_workspace_size(ctypes.byref(d1), 61440) == 0
    d9 = Desc(1, 32, 8, 128, 1, 0.0, 9)          # 9 splits -> 3 blocks per head
    assert lib.nectar_doc_attn_workspace_size(ctypes.byref(d9), 61440) == 8 * 3 * 4 * 520
    dbig = Desc(1, 32, 8, 128, 1, 0.0, 10 ** 6)  # clamped to #tiles (4) -> one block
    assert lib.nectar_doc_attn_workspace_size(ctypes.byref(dbig), 100) == 0
    df = Desc(1, 32, 8, 128, 0, 0.0, 3)          # fp32 path keeps one partial per split
    assert lib.nectar_doc_attn_workspace_size(ctypes.byref(df), 61440) == 8 * 3 * 4 * 520
    loc = Local(1, 1, 513, 513, 512)
    assert lib.nectar_local_workspace_size(ctypes.byref(d), ctypes.byref(loc)) > 0
    m = Module(kind=0, act=0, Ht=4608, Hs=2944)
    assert lib.nectar_module_workspace_size(ctypes.byref(d), ctypes.byref(m)) > 0
    m.kind = 5
    assert lib.nectar_module_workspace_size(ctypes.byref(d), ctypes.byref(m)) == 0


def _mlp_module(Ht=64, Hs=32):
    m = Module(kind=0, act=0, Ht=Ht, Hs=Hs)
    for n in ("W1", "b1", "W2t", "b2", "Ws", "bs", "ws2", "bs2"):
        setattr(m, n, A16)
    return m


def test_module_validation(lib):
    d = Desc(3, 8, 2, 128, 1, 0.0, 0)
    fwd = lambda m, q=A16: lib.nectar_module_forward(ctypes.byref(d), ctypes.byref(m) if m else None,
                                                     q, A16, A16, A16, 0, None)
    assert fwd(None) == EINVAL
    m = _mlp_module(); m.kind = 3
    assert fwd(m) == EINVAL
    m = _mlp_module(); m.act = 9
    assert fwd(m) == EINVAL
    m = _mlp_module(); m.W1 = None
    assert fwd(m) == EINVAL
    m = _mlp_module(); m.Ht = -1
    assert fwd(m) == EINVAL
    m = _mlp_module(); m.bs2 = None
    assert fwd(m) == EINVAL
    m = _mlp_module(); m.W1 = None; m.W2t = None; m.b1 = None; m.Ht = 0
    assert fwd(m, q=None) == EINVAL                                   # q still required
    m = _mlp_module(4608, 2944)
    assert lib.nectar_module_workspace_size(ctypes.byref(d), ctypes.byref(m)) > 0
    assert fwd(m) == EWORKSPACE                                       # 0 bytes given
    kv = Module(kind=1, p=-1)
    assert fwd(kv) == EINVAL
    kv = Module(kind=1, p=100, W=A16, Z=None)
    assert fwd(kv) == EINVAL


def test_local_validation(lib):
    d = Desc(4, 8, 2, 128, 1, 0.0, 0)

    def call(loc, lse=A16, A=A16, dl=None, dA=None, out=None, olse=None, q=A16):
        return lib.nectar_local_attn_lse(ctypes.byref(d), ctypes.byref(loc) if loc else None, q, A16, A16,
                                         lse, A, dl, dA, out, olse, None, 0, None)

    assert call(None) == EINVAL
    assert call(Local(3, 1, 10, 10, 9)) == EINVAL                   # B * Tq != R
    assert call(Local(4, 1, 10, 8, 9)) == EINVAL                    # T_cap < T_loc
    assert call(Local(4, 1, 10, 10, -1)) == EINVAL                  # q_offset
    assert call(Local(4, 1, 10, 10, 9), lse=None, A=None) == EINVAL  # no output requested
    assert call(Local(4, 1, 10, 10, 9), out=A16) == EINVAL          # merge needs the doc pair
    assert call(Local(4, 1, 10, 10, 9), dl=A16, dA=A16) == EINVAL   # doc pair without output
    assert call(Local(4, 1, 10, 10, 9), q=MIS) == EINVAL
    big = Local(4, 1, 5000, 5000, 4999)
    assert lib.nectar_local_workspace_size(ctypes.byref(d), ctypes.byref(big)) > 0
    assert call(big) == EWORKSPACE


def test_workspace_init_validation(lib):
    lib.nectar_workspace_init.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert lib.nectar_workspace_init(None, 0, None) == OK          # nothing to do, no launch
    assert lib.nectar_workspace_init(None, 64, None) == EINVAL
    assert lib.nectar_workspace_init(MIS, 64, None) == EINVAL


def _deep(depth, width, act=1):
    """A well-formed deep module description with fake (aligned) pointers."""
    dm = Deep()
    dm.depth[:] = list(depth)
    dm.width[:] = list(width)
    dm.act = act
    Db, Ds, Dt = depth
    for l in range(min(sum(depth), DEEP_MAX)):
        part = 0 if l < Db else (1 if l < Db + Ds else 2)
        first = (0, Db, Db + Ds)[part]
        reads_state = l > first or (part > 0 and Db > 0)
        dm.Wq[l], dm.b[l] = A16, A16
        dm.Wh[l] = A16 if reads_state else None
    dm.ws_out = dm.bs_out = dm.Wt_out = dm.bt_out = A16
    return dm


def test_deep_module_validation_and_workspace(lib):
    d = Desc(3, 8, 2, 128, 1, 0.0, 0)
    Rp = 3 * 4

    def fwd(dm, q=A16):
        m = Module(kind=2)
        m.deep = ctypes.pointer(dm) if dm is not None else None
        return lib.nectar_module_forward(ctypes.byref(d), ctypes.byref(m), q, A16, A16, A16, 0, None)

    def wsz(dm):
        m = Module(kind=2)
        m.deep = ctypes.pointer(dm)
        return lib.nectar_module_workspace_size(ctypes.byref(d), ctypes.byref(m))

    # two ping-pong bf16 state buffers per part: 2 * (H_b + H_s + H_t) * Hkv * Rp * 2 bytes
    assert wsz(_deep((0, 2, 3), (0, 64, 96))) == 2 * (64 + 96) * 2 * Rp * 2
    assert wsz(_deep((2, 1, 2), (128, 32, 64))) == 2 * (128 + 32 + 64) * 2 * Rp * 2
    assert wsz(_deep((0, 2, 3), (7, 64, 96))) == 2 * (64 + 96) * 2 * Rp * 2    # backbone width unused
    # a workspace below that size is refused before any launch
    assert fwd(_deep((0, 2, 3), (0, 64, 96))) == EWORKSPACE
    assert fwd(None) == EINVAL
    assert fwd(_deep((0, 0, 3), (0, 64, 96))) == EINVAL             # no score network at all
    assert fwd(_deep((0, 2, 0), (0, 64, 96))) == EINVAL             # no target network
    assert fwd(_deep((0, 2, -1), (0, 64, 96))) == EINVAL
    assert fwd(_deep((0, 2, 3), (0, 0, 96))) == EINVAL              # a part with layers needs a width
    assert fwd(_deep((0, 2, 3), (0, 48, 96))) == EUNSUPPORTED       # widths are multiples of 32
    assert fwd(_deep((8, 8, 8), (64, 64, 64))) == EUNSUPPORTED      # more than 16 layers
    assert fwd(_deep((0, 2, 3), (0, 64, 96), act=9)) == EINVAL
    dm = _deep((0, 2, 3), (0, 64, 96))
    dm.Wh[0] = A16                                                  # the first layer reads only q
    assert fwd(dm) == EINVAL
    dm = _deep((0, 2, 3), (0, 64, 96))
    dm.Wh[1] = None                                                 # the second reads the state
    assert fwd(dm) == EINVAL
    dm = _deep((2, 1, 2), (64, 32, 64))
    dm.Wh[2] = None                                                 # a head after a backbone reads it
    assert fwd(dm) == EINVAL
    dm = _deep((0, 2, 3), (0, 64, 96))
    dm.Wq[4] = MIS
    assert fwd(dm) == EINVAL
    dm = _deep((0, 2, 3), (0, 64, 96))
    dm.bt_out = None
    assert fwd(dm) == EINVAL
    assert fwd(_deep((0, 2, 3), (0, 64, 96)), q=MIS) == EINVAL


def test_merge_validation(lib):
    d = Desc(2, 8, 2, 128, 1, 0.0, 0)
    assert lib.nectar_merge(ctypes.byref(d), None, A16, A16, A16, A16, None, None) == EINVAL
    assert lib.nectar_merge(ctypes.byref(d), A16, A16, A16, A16, A16 + 1, None, None) == EINVAL
    assert lib.nectar_merge(None, A16, A16, A16, A16, A16, None, None) == EINVAL
    d0 = Desc(0, 8, 2, 128, 1, 0.0, 0)
    assert lib.nectar_merge(ctypes.byref(d0), None, None, None, None, None, None, None) == OK


def test_merge_k_validation(lib):
    P = ctypes.c_void_p
    d = Desc(2, 8, 2, 128, 1, 0.0, 0)
    arr = lambda *v: (P * max(len(v), 1))(*v)
    two = (arr(A16, A16), arr(A16, A16))
    call = lambda K, pa, pA, lam, Al, out=A16, dd=d: lib.nectar_merge_k(
        ctypes.byref(dd) if dd is not None else None, K, pa, pA, lam, Al, out, None, None)
    assert call(2, *two, A16, A16, dd=None) == EINVAL
    assert call(-1, *two, A16, A16) == EINVAL
    assert call(9, arr(*[A16] * 9), arr(*[A16] * 9), A16, A16) == EINVAL     # above the maximum of 8
    assert call(2, *two, A16, None) == EINVAL                                 # lam without A_loc
    assert call(2, *two, None, A16) == EINVAL
    assert call(0, None, None, None, None) == EINVAL                          # no pair at all
    assert call(2, None, None, A16, A16) == EINVAL
    assert call(2, arr(A16, A16 + 2), arr(A16, A16), A16, A16) == EINVAL     # misaligned logit
    assert call(2, *two, A16, A16, out=A16 + 1) == EINVAL
    assert call(2, *two, A16, A16, out=None) == EINVAL
    d0 = Desc(0, 8, 2, 128, 1, 0.0, 0)
    assert call(2, *two, None, None, out=None, dd=d0) == OK                  # no rows: a no-op


def test_fit_metrics_validation(lib):
    d = Desc(2, 8, 2, 128, 1, 0.0, 0)
    call = lambda dd=d, q=A16, a=A16, A=A16, al=A16, Ae=A16, row=A16, head=A16, ws=A16, wsb=1 << 20: \
        lib.nectar_fit_metrics(ctypes.byref(dd) if dd is not None else None, q, a, A, al, Ae, row, head, ws, wsb,
                               None)
    need = lib.nectar_fit_metrics_workspace_size(ctypes.byref(d))
    assert need == 2 * 64 * 3 * 8
    assert call(wsb=need - 1) == EWORKSPACE
    assert call(dd=None) == EINVAL
    assert call(q=MIS) == EINVAL
    assert call(A=A16 + 4) == EINVAL            # d-vectors are 16-byte aligned
    assert call(Ae=None) == EINVAL
    assert call(row=None) == EINVAL
    assert call(head=A16 + 4) == EINVAL          # fp64 sums
    assert call(dd=Desc(2, 8, 2, 96, 1, 0.0, 0)) == EUNSUPPORTED
    assert call(dd=Desc(0, 8, 2, 128, 1, 0.0, 0), q=None, a=None, A=None, al=None, Ae=None, row=None) == OK


def test_training_entry_points_validation(lib):
    d = Desc(5, 8, 2, 128, 1, 0.0, 0)
    m = _mlp_module(96, 64)
    n = lib.nectar_mlp_param_count(ctypes.byref(d), ctypes.byref(m))
    assert n == 2 * (2 * 96 * 128 + 96 + 128 + 64 * 128 + 2 * 64 + 1)
    ws = lib.nectar_mlp_train_workspace_size(ctypes.byref(d), ctypes.byref(m))
    assert ws > 0
    lg = lambda dd=d, mm=m, wsb=ws, grad=A16, la=0.1: lib.nectar_mlp_loss_grad(
        ctypes.byref(dd), ctypes.byref(mm), A16, A16, A16, la, 1.0, grad, A16, A16, wsb, None)
    assert lg(wsb=ws - 1) == EWORKSPACE
    assert lg(grad=A16 + 4) == EINVAL
    assert lg(la=float("nan")) == EINVAL
    assert lg(dd=Desc(5, 8, 2, 128, 0, 0.0, 0)) == EUNSUPPORTED           # fp32 modules
    assert lg(mm=_mlp_module(100, 64)) == EUNSUPPORTED                          # widths are multiples of 32
    assert lg(mm=_mlp_module(96, 0)) == EUNSUPPORTED
    assert lg(mm=Module(kind=1, p=10, W=A16, Z=A16)) == EUNSUPPORTED      # Quadrature: not this step
    assert lg(dd=Desc(0, 8, 2, 128, 1, 0.0, 0)) == EINVAL                # needs rows
    hp = HP(0.1, 1.0, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1.0, 1)
    ad = lambda h, nn=10, th=A16: lib.nectar_adamw_step(nn, th, A16, A16, A16, ctypes.byref(h), None)
    assert ad(hp, nn=0) == OK
    assert ad(hp, nn=-1) == EINVAL
    assert ad(hp, th=A16 + 2) == EINVAL
    for bad in (HP(0.1, 1.0, 1e-4, 1.0, 0.999, 1e-8, 0.0, 1.0, 1), HP(0.1, 1.0, 1e-4, 0.9, 0.999, 0.0, 0.0, 1.0, 1),
                HP(0.1, 1.0, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1.0, 0), HP(0.1, 1.0, float("inf"), 0.9, 0.999, 1e-8, 0.0,
                                                                    1.0, 1)):
        assert ad(bad) == EINVAL
    ts = lambda h=hp, wsb=ws, th=A16: lib.nectar_mlp_train_step(
        ctypes.byref(d), ctypes.byref(m), A16, A16, A16, ctypes.byref(h), th, A16, A16, A16, None, None, A16, wsb,
        None)
    assert ts(wsb=ws - 1) == EWORKSPACE
    assert ts(th=A16 + 4) == EINVAL
    assert ts(h=HP(0.1, 1.0, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1.0, 0)) == EINVAL


def test_oracle_and_product_share_no_code():
    """The oracle is its own C file; the HIP sources never include or name it."""
    csrc = os.path.join(ROOT, "learned_kv_cache_02_amd", "csrc")
    for f in os.listdir(csrc):
        txt = open(os.path.join(csrc, f)).read()
        assert "oracle" not in txt.lower(), f
    for f in ("nectar.py", "build_native.py", "__init__.py"):
        txt = open(os.path.join(ROOT, "learned_kv_cache_02_amd", f)).read()
        assert "import oracle" not in txt and "from oracle" not in txt, f


def test_layer_step_validation(lib):
    d = Desc(1, 32, 8, 128, 1, 0.0, 0)
    loc = Local(1, 1, 513, 513, 512)
    m = _mlp_module(4608, 2944)

    def call(outs, module=None, n=61440, ws=None, nbytes=0, q=A16, k=A16, lc=loc, desc=d):
        return lib.nectar_layer_step(ctypes.byref(desc), n, ctypes.byref(lc) if lc else None, q, k, A16, A16,
                                     A16, ctypes.byref(module) if module else None,
                                     ctypes.byref(outs) if outs else None, ws, nbytes, None)

    both = StepOuts(out_exact=A16, lse_exact=A16, out_nectar=A16, lse_nectar=A16)
    exact_only = StepOuts(out_exact=A16, lse_exact=A16)
    assert call(None) == EINVAL                                        # no output struct
    assert call(StepOuts()) == EINVAL                                  # nothing requested
    assert call(both) == EINVAL                                        # Nectar outputs without a module
    assert call(exact_only, module=m) == EINVAL                        # module without Nectar outputs
    assert call(both, module=m, lc=None) == EINVAL
    assert call(both, module=m, lc=Local(2, 1, 513, 513, 512)) == EINVAL     # B * Tq != R
    assert call(both, module=m, n=-1) == EINVAL
    assert call(StepOuts(out_exact=A16 + 1), module=None) == EINVAL    # misaligned bf16 output
    assert call(exact_only, q=MIS) == EINVAL
    assert call(exact_only, k=None) == EINVAL                          # exact output needs the cache
    bad = _mlp_module(); bad.act = 7
    assert call(both, module=bad) == EINVAL
    need = lib.nectar_layer_step_workspace_size(ctypes.byref(d), 61440, ctypes.byref(loc), ctypes.byref(m), 1)
    # deferred partials of all three parts: the document's 58 blocks per head (464 of the 512
    # two-per-CU block slots, leaving room for the module's blocks) and the local part's 3
    # (4 rows x 520 B each), plus the module's split partials
    assert need >= 8 * 58 * 4 * 520 + 8 * 3 * 4 * 520
    assert call(both, module=m, ws=A16, nbytes=need - 1) == EWORKSPACE
    only_loc = lib.nectar_layer_step_workspace_size(ctypes.byref(d), 61440, ctypes.byref(loc), None, 0)
    assert 0 < only_loc < need
    assert lib.nectar_layer_step_workspace_size(None, 61440, ctypes.byref(loc), None, 1) == 0
    d0 = Desc(0, 32, 8, 128, 1, 0.0, 0)                                # R == 0: valid no-op
    assert call(exact_only, desc=d0, lc=Local(0, 1, 513, 513, 512), q=None) == OK


def test_layer_step_static_validation(lib):
    """The allocation-free layer step validates on the host before any HIP call:
    argument errors, and plans larger than its static device scratch
    (NECTAR_STATIC_SCRATCH_BYTES = 64 MiB), are rejected without a GPU."""
    P, D = ctypes.c_void_p, ctypes.POINTER(Desc)
    f = lib.nectar_layer_step_static
    f.argtypes = [D, ctypes.c_int64, ctypes.POINTER(Local), P, P, P, P, P, ctypes.POINTER(Module),
                  ctypes.POINTER(StepOuts), P]
    static_bytes = 64 << 20
    hdr = open(HDR).read()
    assert "#define NECTAR_STATIC_SCRATCH_BYTES (64u << 20)" in hdr

    def call(desc, n, lc, module, outs, q=A16):
        return f(ctypes.byref(desc), n, ctypes.byref(lc), q, A16, A16, A16, A16,
                 ctypes.byref(module) if module else None, ctypes.byref(outs), None)

    both = StepOuts(out_exact=A16, lse_exact=A16, out_nectar=A16, lse_nectar=A16)
    # the 16 x 1,024-token prefill layer with the rho = 10 % module: far beyond the scratch
    dp = Desc(16 * 1024, 28, 4, 128, 1, 0.0, 0)
    lp = Local(16, 1024, 1024, 1024, 0)
    mp = _mlp_module(7680, 5120)
    need = lib.nectar_layer_step_workspace_size(ctypes.byref(dp), 131072, ctypes.byref(lp), ctypes.byref(mp), 1)
    assert need > static_bytes
    assert call(dp, 131072, lp, mp, both) == EWORKSPACE
    # argument errors come first, as in nectar_layer_step
    assert call(dp, 131072, lp, mp, both, q=MIS) == EINVAL
    assert call(dp, -1, lp, mp, both) == EINVAL
    # the decode shapes fit: the 4B layer with both paths needs a few MiB
    d = Desc(1, 32, 8, 128, 1, 0.0, 0)
    loc = Local(1, 1, 513, 513, 512)
    m = _mlp_module(4608, 2944)
    assert 0 < lib.nectar_layer_step_workspace_size(ctypes.byref(d), 61440, ctypes.byref(loc), ctypes.byref(m),
                                                    1) <= static_bytes


def test_doc_attn_two_pass_validation(lib):
    P = ctypes.c_void_p
    D = ctypes.POINTER(Desc)
    lib.nectar_doc_attn_partials_size.argtypes = [D, ctypes.c_int64]
    lib.nectar_doc_attn_partials_size.restype = ctypes.c_size_t
    lib.nectar_doc_attn_partials.argtypes = [D, ctypes.c_int64, P, P, P, P, ctypes.c_size_t, P]
    lib.nectar_doc_attn_combine.argtypes = [D, ctypes.c_int64, P, ctypes.c_size_t, P, P, P]
    d = Desc(1, 32, 8, 128, 1, 0.0, 0)
    # same plan as the one-call form: 64 partials per row, 4 rows per head, 520 B each
    assert lib.nectar_doc_attn_partials_size(ctypes.byref(d), 61440) == 8 * 64 * 4 * 520
    d1 = Desc(1, 32, 8, 128, 1, 0.0, 1)          # one split: still one partial per row
    assert lib.nectar_doc_attn_partials_size(ctypes.byref(d1), 61440) == 8 * 1 * 4 * 520
    assert lib.nectar_doc_attn_partials_size(ctypes.byref(d), 0) == 0
    need = lib.nectar_doc_attn_partials_size(ctypes.byref(d), 61440)
    assert lib.nectar_doc_attn_partials(ctypes.byref(d), 61440, A16, A16, A16, A16, need - 1, None) == EWORKSPACE
    assert lib.nectar_doc_attn_partials(ctypes.byref(d), 61440, MIS, A16, A16, A16, need, None) == EINVAL
    assert lib.nectar_doc_attn_partials(ctypes.byref(d), -1, A16, A16, A16, A16, need, None) == EINVAL
    assert lib.nectar_doc_attn_combine(ctypes.byref(d), 61440, A16, need - 1, A16, A16, None) == EWORKSPACE
    assert lib.nectar_doc_attn_combine(ctypes.byref(d), 61440, A16, need, None, A16, None) == EINVAL
    assert lib.nectar_doc_attn_combine(ctypes.byref(d), 61440, MIS, need, A16, A16, None) == EINVAL
