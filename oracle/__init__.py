"""CPU oracle for the MoE-layer forward pass -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It wraps moe_oracle.c (plain C, fp64 accumulation; see the
header of that file for what it computes and how each step is pinned) through
ctypes.  Inputs are duck-typed layer objects holding numpy arrays (attributes
router_w, router_b, gate/up/down and sh_* with codes, scales, tensor_scale);
nothing here depends on the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")  # override: an instrumented build
_FMT = {"bf16": 0, "q4_1": 1, "nvfp4": 2}

_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Mat(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("dm", ctypes.c_void_p), ("e4m3", ctypes.c_void_p),
                ("ts", ctypes.c_void_p)]


class _Layer(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("f", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("renorm", ctypes.c_int32), ("shared_scale", ctypes.c_double),
                ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("gate", _Mat), ("up", _Mat), ("down", _Mat),
                ("sh_gate", _Mat), ("sh_up", _Mat), ("sh_down", _Mat)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        vp, i32, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        for name in ("orc_fp16_value", "orc_bf16_value"):
            getattr(L, name).restype = dbl
            getattr(L, name).argtypes = [ctypes.c_uint16]
        for name in ("orc_e4m3_value", "orc_e2m1_value"):
            getattr(L, name).restype = dbl
            getattr(L, name).argtypes = [ctypes.c_uint8]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_bf16_rne.argtypes = [dbl]
        L.orc_weight.restype = ctypes.c_float
        L.orc_weight.argtypes = [ctypes.POINTER(_Mat), ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        L.orc_decode_matrix.argtypes = [ctypes.POINTER(_Mat), ctypes.c_int64, ctypes.c_void_p]
        L.orc_decode_matrix.restype = None
        L.orc_topk.argtypes = [vp, i32, i32, vp, vp]
        L.orc_route_weights.argtypes = [vp, i32, vp, i32, i32, vp]
        L.orc_layer_forward.argtypes = [ctypes.POINTER(_Layer), vp, i32, vp, vp, vp, vp, vp, vp, i32]
        L.orc_route.argtypes = [ctypes.POINTER(_Layer), vp, i32, vp, vp, vp, vp, i32]
        L.orc_buckets.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        L.orc_rmsnorm_bf16.argtypes = [vp, i32, dbl, vp]
        L.orc_stack_forward.argtypes = [vp, i32, vp, i32, dbl, vp, vp, vp, vp, i32]
        L.orc_expert.argtypes = [ctypes.POINTER(_Layer), ctypes.POINTER(_Mat), ctypes.POINTER(_Mat),
                                 ctypes.POINTER(_Mat), ctypes.c_int64, vp, vp]
        L.orc_max_threads.restype = i32
        L.orc_head_logits.argtypes = [ctypes.POINTER(_Mat), vp, i32, vp, i32, vp, i32]
        L.orc_attn_prep.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, i32, dbl, dbl, vp, vp]
        L.orc_attn_decode.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _mat(q, keep):
    m = _Mat()
    if q is None:
        return m
    m.fmt, m.rows, m.cols = _FMT[q.fmt], q.rows, q.cols
    codes = np.ascontiguousarray(q.codes)
    keep.append(codes)
    m.codes = codes.ctypes.data
    if q.fmt == "q4_1":
        s = np.ascontiguousarray(q.scales, np.uint16)
        keep.append(s)
        m.dm = s.ctypes.data
    elif q.fmt == "nvfp4":
        s = np.ascontiguousarray(q.scales, np.uint8)
        t = np.ascontiguousarray(q.tensor_scale, np.float32)
        keep += [s, t]
        m.e4m3, m.ts = s.ctypes.data, t.ctypes.data
    return m


class OracleLayer:
    """ctypes view of a layer object; holds references to the arrays it points at."""

    def __init__(self, layer):
        self.keep = []
        s = _Layer()
        s.d, s.E, s.k, s.f = layer.d, layer.E, layer.k, layer.f
        s.n_shared, s.renorm, s.shared_scale = layer.n_shared, layer.renorm, float(layer.shared_scale)
        rw = np.ascontiguousarray(layer.router_w, np.uint16)
        self.keep.append(rw)
        s.router_w = rw.ctypes.data
        if layer.router_b is not None:
            rb = np.ascontiguousarray(layer.router_b, np.float32)
            self.keep.append(rb)
            s.router_b = rb.ctypes.data
        for name in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
            setattr(s, name, _mat(getattr(layer, name, None), self.keep))
        self.s = s
        self.layer = layer

    @property
    def ref(self):
        return ctypes.byref(self.s)


def _ol(layer):
    return layer if isinstance(layer, OracleLayer) else OracleLayer(layer)


# ---- scalar decoders (pins) ------------------------------------------------------

def fp16_value(h: int) -> float:
    return lib().orc_fp16_value(h)


def bf16_value(b: int) -> float:
    return lib().orc_bf16_value(b)


def e4m3_value(b: int) -> float:
    return lib().orc_e4m3_value(b)


def e2m1_value(c: int) -> float:
    return lib().orc_e2m1_value(c)


def bf16_rne(v: float) -> int:
    return int(lib().orc_bf16_rne(v))


def weight(q, n: int, r: int, c: int) -> float:
    keep = []
    m = _mat(q, keep)
    return lib().orc_weight(ctypes.byref(m), n, r, c)


def decode_matrix(q, n: int) -> np.ndarray:
    """All weights of matrix n of a stored set, decoded to fp32."""
    keep = []
    m = _mat(q, keep)
    out = np.empty((q.rows, q.cols), np.float32)
    lib().orc_decode_matrix(ctypes.byref(m), n, _p(out))
    return out


# ---- steps -------------------------------------------------------------------------

def topk(logits: np.ndarray, k: int):
    lg = np.ascontiguousarray(logits, np.float64)
    ids = np.empty(k, np.int32)
    gap = np.zeros(1, np.float64)
    lib().orc_topk(_p(lg), lg.size, k, _p(ids), _p(gap))
    return ids, float(gap[0])


def route_weights(logits: np.ndarray, ids: np.ndarray, renorm: int = 1) -> np.ndarray:
    lg = np.ascontiguousarray(logits, np.float64)
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.empty(ids.size, np.float64)
    lib().orc_route_weights(_p(lg), lg.size, _p(ids), ids.size, renorm, _p(w))
    return w


def layer_forward(layer, x: np.ndarray, forced_ids: np.ndarray | None = None, threads: int = 0):
    """x: bf16 bits [T][d].  Returns dict(out fp64 [T][d], ids [T][k], w [T][k],
    logits [T][E], gaps [T])."""
    L = _ol(layer)
    x = np.ascontiguousarray(x, np.uint16)
    T = x.shape[0]
    s = L.s
    out = np.empty((T, s.d), np.float64)
    ids = np.empty((T, s.k), np.int32)
    w = np.empty((T, s.k), np.float64)
    logits = np.empty((T, s.E), np.float64)
    gaps = np.empty(T, np.float64)
    fi = None if forced_ids is None else np.ascontiguousarray(forced_ids, np.int32)
    if T > 0:
        lib().orc_layer_forward(L.ref, _p(x), T, _p(fi), _p(out), _p(ids), _p(w), _p(logits), _p(gaps), threads)
    return dict(out=out, ids=ids, w=w, logits=logits, gaps=gaps)


def route(layer, x: np.ndarray, threads: int = 0):
    """Routing only: dict(ids, w, logits, gaps)."""
    L = _ol(layer)
    x = np.ascontiguousarray(x, np.uint16)
    T = x.shape[0]
    s = L.s
    ids = np.empty((T, s.k), np.int32)
    w = np.empty((T, s.k), np.float64)
    logits = np.empty((T, s.E), np.float64)
    gaps = np.empty(T, np.float64)
    if T > 0:
        lib().orc_route(L.ref, _p(x), T, _p(ids), _p(w), _p(logits), _p(gaps), threads)
    return dict(ids=ids, w=w, logits=logits, gaps=gaps)


def expert(layer, which: str, n: int, x: np.ndarray) -> np.ndarray:
    """One expert on one fp64 row; which = 'routed' or 'shared'."""
    L = _ol(layer)
    xd = np.ascontiguousarray(x, np.float64)
    y = np.empty(L.s.d, np.float64)
    if which == "routed":
        mats = (L.s.gate, L.s.up, L.s.down)
    else:
        mats = (L.s.sh_gate, L.s.sh_up, L.s.sh_down)
    lib().orc_expert(L.ref, *[ctypes.byref(m) for m in mats], n, _p(xd), _p(y))
    return y


def buckets(ids: np.ndarray, E: int):
    """ids [T][k] -> dict(counts [E], offsets [E+1], perm [T*k], inv_perm [T*k])."""
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    S = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(max(S, 1), np.int32)
    inv = np.empty(max(S, 1), np.int32)
    lib().orc_buckets(_p(ids), T, k, E, _p(counts), _p(offsets), _p(perm), _p(inv))
    return dict(counts=counts, offsets=offsets, perm=perm[:S], inv_perm=inv[:S])


def rmsnorm_bf16(r: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    r = np.ascontiguousarray(r, np.float64)
    out = np.empty(r.size, np.uint16)
    lib().orc_rmsnorm_bf16(_p(r), r.size, eps, _p(out))
    return out


def stack_forward(layers, x: np.ndarray, eps: float = 1e-6, threads: int = 0, record: bool = True):
    """x: bf16 bits [T][d].  Returns dict(out bf16 [T][d], and if record:
    xin [L][T][d] bf16, yout [L][T][d] bf16, ids [L][T][k])."""
    Ls = [_ol(l) for l in layers]
    arr = (ctypes.POINTER(_Layer) * len(Ls))(*[ctypes.pointer(l.s) for l in Ls])
    x = np.ascontiguousarray(x, np.uint16)
    T, d = x.shape
    nl = len(Ls)
    k = Ls[0].s.k
    out = np.empty((T, d), np.uint16)
    xin = np.empty((nl, T, d), np.uint16) if record else None
    yout = np.empty((nl, T, d), np.uint16) if record else None
    ids = np.empty((nl, T, k), np.int32) if record else None
    lib().orc_stack_forward(ctypes.cast(arr, ctypes.c_void_p), nl, _p(x), T, eps, _p(out), _p(xin), _p(yout),
                            _p(ids), threads)
    return dict(out=out, xin=xin, yout=yout, ids=ids)


def head_logits(q, x: np.ndarray, rows: np.ndarray | None = None, threads: int = 0) -> np.ndarray:
    """Output-head logits of bf16 tokens x [T][cols] against stored matrix 0 of
    q ([vocab][cols]): fp64 [T][len(rows)] (rows None = every vocabulary row)."""
    keep = []
    m = _mat(q, keep)
    x = np.ascontiguousarray(x, np.uint16)
    T = x.shape[0]
    r = None if rows is None else np.ascontiguousarray(rows, np.int32)
    n = q.rows if r is None else r.size
    out = np.empty((T, n), np.float64)
    if T > 0 and n > 0:
        lib().orc_head_logits(ctypes.byref(m), _p(x), T, _p(r), n, _p(out), threads)
    return out


def attn_prep(q: np.ndarray, k: np.ndarray, q_gain: np.ndarray, k_gain: np.ndarray, pos: np.ndarray, rope: bool,
              theta: float = 10000.0, eps: float = 1e-6):
    """The new token's q [B][HQ][D] and k [B][HK][D] (bf16 bits) normalised per
    head, rotated if `rope`, rounded to bf16: returns (q', k') as bf16 bits."""
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    B, HQ, D = q.shape
    HK = k.shape[1]
    qo, ko = np.empty_like(q), np.empty_like(k)
    g1, g2 = np.ascontiguousarray(q_gain, np.uint16), np.ascontiguousarray(k_gain, np.uint16)
    p = np.ascontiguousarray(pos, np.int32)
    lib().orc_attn_prep(_p(q), _p(k), B, HQ, HK, D, _p(g1), _p(g2), _p(p), int(rope), theta, eps, _p(qo), _p(ko))
    return qo, ko


def attn_decode(q: np.ndarray, kc: np.ndarray, vc: np.ndarray, lens: np.ndarray, window: int,
                sinks: np.ndarray | None, threads: int = 0) -> np.ndarray:
    """Attention of one token per sequence: q [B][HQ][D], caches [B][cap][HK][D]
    (bf16 bits), lens [B]; window 0 = full.  Returns fp64 [B][HQ][D]."""
    q = np.ascontiguousarray(q, np.uint16)
    kc = np.ascontiguousarray(kc, np.uint16)
    vc = np.ascontiguousarray(vc, np.uint16)
    B, HQ, D = q.shape
    cap, HK = kc.shape[1], kc.shape[2]
    ln = np.ascontiguousarray(lens, np.int32)
    sk = None if sinks is None else np.ascontiguousarray(sinks, np.float32)
    out = np.empty((B, HQ, D), np.float64)
    if B > 0:
        lib().orc_attn_decode(_p(q), _p(kc), _p(vc), _p(ln), B, HQ, HK, D, cap, window, _p(sk), _p(out), threads)
    return out


def max_threads() -> int:
    return int(lib().orc_max_threads())
