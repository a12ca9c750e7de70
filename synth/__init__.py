"""Seeded synthetic inputs for the MoE-layer path.

Draws activations, router weights, the optional Zipf router bias and expert
weights, and stores expert weights in the library's layouts (q4_1, NVFP4,
bf16).  It holds no forward arithmetic; the oracle and the HIP library both
read the arrays it returns and neither imports the other.

Recipe (all draws are SplitMix64 streams keyed by (seed, tag, a, b), normals by
Box-Muller; see synth.c):
  * activations  x  ~ bf16(fp32(N(0, 1)))                  key (xseed, X, 0, 0)
  * router       Wr ~ bf16(fp32(N(0, 0.02)))  [E][d]        key (seed, ROUTER, 0, 0)
  * router bias  b[e] = fp32(-s * ln(1 + pi(e))), pi a random permutation of
                 the expert ids (Zipf(s) over a random ranking)  key (seed, BIAS, 0, 0)
  * expert e, matrix j (0 gate [f][d], 1 up [f][d], 2 down [d][f]):
                 fp32(N(0, 0.02)), then the format's encoder   key (seed, EXPERT, e, j)
    the shared expert uses e = SHARED_ID.
  * decode attention: new-token q [B][32][128], k and v [B][4][128], cached keys
                 and values [B][cap][4][128] ~ bf16(fp32(N(0, 1))); q/k RMSNorm gains
                 bf16(1 + N(0, 0.1)) [128]; sinks fp32(N(0, 1)) [32]   key (seed, ATTN, i, 0)
  * output head  W  ~ fp32(N(0, 0.02)) [V][d], then the format's encoder
                 key (seed, HEAD, 0, 0); the vocabulary V is synthetic (the
                 pages do not give it; about 150 k)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.environ.get("MOE_SYNTH_LIB") or os.path.join(_HERE, "libsynth.so")  # override: an instrumented build

TAG_X, TAG_ROUTER, TAG_BIAS, TAG_EXPERT, TAG_HEAD, TAG_ATTN, TAG_EDGE = 1, 2, 3, 4, 5, 6, 7
HEAD_VOCAB = 151552  # synthetic vocabulary of the output-head workload
SHARED_ID = 1_000_000
FMT_CODE = {"bf16": 0, "q4_1": 1, "nvfp4": 2}

_lib = None


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64, u64, u64]
        L.synth_u64.restype = u64
        L.synth_u64.argtypes = [u64, u64]
        L.synth_normal_f32.argtypes = [u64, dbl, vp, i64]
        L.synth_normal_bf16.argtypes = [u64, dbl, vp, i64]
        L.synth_permutation.argtypes = [u64, vp, ctypes.c_int32]
        L.synth_bytes.argtypes = [u64, vp, i64]
        L.synth_q4_1_encode.argtypes = [vp, i64, i64, vp, vp]
        L.synth_nvfp4_encode.argtypes = [vp, i64, i64, vp, vp, vp]
        L.synth_f32_to_bf16.argtypes = [vp, vp, i64]
        L.synth_matrix.argtypes = [u64, dbl, ctypes.c_int, i64, i64, vp, vp, vp]
        L.synth_f64_to_f16.restype = ctypes.c_uint16
        L.synth_f64_to_f16.argtypes = [dbl]
        L.synth_f64_to_e4m3_sat.restype = ctypes.c_uint8
        L.synth_f64_to_e4m3_sat.argtypes = [dbl]
        L.synth_f64_to_e2m1.restype = ctypes.c_uint8
        L.synth_f64_to_e2m1.argtypes = [dbl]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def key(seed: int, tag: int, a: int = 0, b: int = 0) -> int:
    return int(lib().synth_key(seed, tag, a, b))


# ---- raw draws --------------------------------------------------------------

def normal_f32(k: int, sigma: float, n: int) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normal_f32(k, sigma, _p(out), n)
    return out


def normal_bf16(k: int, sigma: float, n: int) -> np.ndarray:
    out = np.empty(n, np.uint16)
    lib().synth_normal_bf16(k, sigma, _p(out), n)
    return out


def uniform_bytes(k: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint8)
    lib().synth_bytes(k, _p(out), n)
    return out


def permutation(k: int, n: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().synth_permutation(k, _p(out), n)
    return out


# ---- encoders (arrays in, packed arrays out) ------------------------------------

def encode_q4_1(w: np.ndarray):
    """w: fp32 [rows][cols] -> (codes u8 [rows][cols/2], dm fp16-bits u16 [rows][cols/32][2])."""
    w = np.ascontiguousarray(w, np.float32)
    rows, cols = w.shape
    assert cols % 32 == 0
    codes = np.empty((rows, cols // 2), np.uint8)
    dm = np.empty((rows, cols // 32, 2), np.uint16)
    lib().synth_q4_1_encode(_p(w), rows, cols, _p(codes), _p(dm))
    return codes, dm


def encode_nvfp4(w: np.ndarray):
    """w: fp32 [rows][cols] -> (codes u8 [rows][cols/2], scales u8 [rows][cols/16], ts fp32)."""
    w = np.ascontiguousarray(w, np.float32)
    rows, cols = w.shape
    assert cols % 16 == 0
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    ts = np.zeros(1, np.float32)
    lib().synth_nvfp4_encode(_p(w), rows, cols, _p(codes), _p(scales), _p(ts))
    return codes, scales, float(ts[0])


def encode_bf16(w: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w, np.float32)
    out = np.empty(w.shape, np.uint16)
    lib().synth_f32_to_bf16(_p(w), _p(out), w.size)
    return out


# ---- layer containers ---------------------------------------------------------

@dataclass
class QMat:
    """A stored matrix set [n][rows][cols] in one format.

    codes : q4_1/nvfp4 u8 [n][rows][cols/2]; bf16 u16 [n][rows][cols]
    scales: q4_1 u16 (fp16 bits) [n][rows][cols/32][2] = {d, m};
            nvfp4 u8 (E4M3) [n][rows][cols/16]; bf16 None.  Within a row the
            32-element blocks' scales are stored in the order k mod 16, then
            k // 16 (where 16 divides the block count; NVFP4 keeps a block's
            two scales together)
    tensor_scale: nvfp4 fp32 [n]; else None
    """
    fmt: str
    n: int
    rows: int
    cols: int
    codes: np.ndarray
    scales: np.ndarray | None = None
    tensor_scale: np.ndarray | None = None

    def nbytes(self, count: int = 1) -> int:
        """Stored bytes of `count` matrices of this set."""
        per = self.rows * self.cols
        if self.fmt == "bf16":
            return count * per * 2
        if self.fmt == "q4_1":
            return count * (per // 2 + per // 32 * 4)
        return count * (per // 2 + per // 16 + 4)


def alloc_qmat(fmt: str, n: int, rows: int, cols: int) -> QMat:
    if fmt == "bf16":
        return QMat(fmt, n, rows, cols, np.empty((n, rows, cols), np.uint16))
    if fmt == "q4_1":
        return QMat(fmt, n, rows, cols, np.empty((n, rows, cols // 2), np.uint8),
                    np.empty((n, rows, cols // 32, 2), np.uint16))
    if fmt == "nvfp4":
        return QMat(fmt, n, rows, cols, np.empty((n, rows, cols // 2), np.uint8),
                    np.empty((n, rows, cols // 16), np.uint8), np.zeros(n, np.float32))
    raise ValueError(fmt)


def fill_matrix(q: QMat, i: int, k: int, sigma: float) -> None:
    """Draw matrix i of q from stream k (N(0, sigma)) and encode it in place."""
    codes = q.codes[i]
    scales = q.scales[i] if q.scales is not None else None
    ts = q.tensor_scale[i:i + 1] if q.tensor_scale is not None else None
    lib().synth_matrix(k, sigma, FMT_CODE[q.fmt], q.rows, q.cols, _p(codes),
                       _p(scales) if scales is not None else None,
                       _p(ts) if ts is not None else None)


@dataclass
class Layer:
    fmt: str
    d: int
    E: int
    k: int
    f: int
    n_shared: int
    shared_scale: float
    renorm: int
    router_w: np.ndarray                 # u16 bf16 bits [E][d]
    router_b: np.ndarray | None          # fp32 [E] or None
    gate: QMat
    up: QMat
    down: QMat
    sh_gate: QMat | None = None
    sh_up: QMat | None = None
    sh_down: QMat | None = None
    meta: dict = field(default_factory=dict)

    def expert_bytes(self) -> int:
        return self.gate.nbytes() + self.up.nbytes() + self.down.nbytes()


def make_layer(seed: int = 0, fmt: str = "q4_1", E: int = 256, d: int = 2048, f: int = 512, k: int = 6,
               n_shared: int = 1, shared_scale: float = 1.0, zipf: float | None = None, renorm: int = 1,
               sigma: float = 0.02, router_sigma: float = 0.02) -> Layer:
    """One MoE layer drawn from `seed` (see the module recipe)."""
    router_w = normal_bf16(key(seed, TAG_ROUTER), router_sigma, E * d).reshape(E, d)
    router_b = None
    if zipf is not None:
        pi = permutation(key(seed, TAG_BIAS), E)
        router_b = (-zipf * np.log1p(pi.astype(np.float64))).astype(np.float32)
    gate, up, down = alloc_qmat(fmt, E, f, d), alloc_qmat(fmt, E, f, d), alloc_qmat(fmt, E, d, f)
    for e in range(E):
        fill_matrix(gate, e, key(seed, TAG_EXPERT, e, 0), sigma)
        fill_matrix(up, e, key(seed, TAG_EXPERT, e, 1), sigma)
        fill_matrix(down, e, key(seed, TAG_EXPERT, e, 2), sigma)
    L = Layer(fmt, d, E, k, f, n_shared, shared_scale, renorm, router_w, router_b, gate, up, down,
              meta=dict(seed=seed, zipf=zipf))
    if n_shared:
        L.sh_gate, L.sh_up, L.sh_down = alloc_qmat(fmt, 1, f, d), alloc_qmat(fmt, 1, f, d), alloc_qmat(fmt, 1, d, f)
        fill_matrix(L.sh_gate, 0, key(seed, TAG_EXPERT, SHARED_ID, 0), sigma)
        fill_matrix(L.sh_up, 0, key(seed, TAG_EXPERT, SHARED_ID, 1), sigma)
        fill_matrix(L.sh_down, 0, key(seed, TAG_EXPERT, SHARED_ID, 2), sigma)
    return L


def make_x(T: int, d: int = 2048, xseed: int = 0, sigma: float = 1.0) -> np.ndarray:
    """bf16 bits [T][d] of fp32(N(0, sigma))."""
    return normal_bf16(key(xseed, TAG_X), sigma, T * d).reshape(T, d)


def make_head(V: int = HEAD_VOCAB, fmt: str = "q4_1", seed: int = 0, d: int = 2048, sigma: float = 0.02) -> QMat:
    """Output-head matrix [V][d] (one stored matrix) drawn from `seed`."""
    q = alloc_qmat(fmt, 1, V, d)
    fill_matrix(q, 0, key(seed, TAG_HEAD), sigma)
    return q


ATTN_HQ, ATTN_HK, ATTN_D = 32, 4, 128  # query heads, key-value heads, head dimension
ATTN_WINDOW = 513                        # sliding window: the current token and the 512 before it


def make_attn(B: int, cap: int, seed: int = 0, HQ: int = ATTN_HQ, HK: int = ATTN_HK, D: int = ATTN_D) -> dict:
    """Inputs of one decode-attention step: the new token's q, k, v (bf16 bits),
    a cache of `cap` positions per sequence in the plain layout [B][cap][HK][D]
    (keys as stored: already normalised and rotated), the gains and the sinks."""
    def bf(i, n, sigma=1.0):
        return normal_bf16(key(seed, TAG_ATTN, i), sigma, n)
    g = normal_f32(key(seed, TAG_ATTN, 5), 0.1, 2 * D) + np.float32(1.0)
    return dict(q=bf(0, B * HQ * D).reshape(B, HQ, D), k=bf(1, B * HK * D).reshape(B, HK, D),
                v=bf(2, B * HK * D).reshape(B, HK, D),
                k_cache=bf(3, B * cap * HK * D).reshape(B, cap, HK, D),
                v_cache=bf(4, B * cap * HK * D).reshape(B, cap, HK, D),
                q_gain=encode_bf16(g[:D]), k_gain=encode_bf16(g[D:]),
                sinks=normal_f32(key(seed, TAG_ATTN, 6), 1.0, HQ))


# ---- patterned weights and activations for edge cases ------------------------------------
# Codes and scales are written directly (uniform random bytes, or bit patterns),
# not drawn as numbers and encoded, so that every stored code occurs.

# NVFP4 scale bytes: the 8 consecutive E4M3 codes from each base together cover
# every finite code of both signs (0x7F and 0xFF are NaN and never written).
E4M3_BASES = [8 * i for i in range(15)] + [0x77] + [0x80 | (8 * i) for i in range(15)] + [0xF7]
Q4_1_REGIMES = ("mixed", "subnormal", "large", "normal", "small_positive")


def _e4m3_binade(b: int) -> int:
    """floor(log2 |value|) of an E4M3 code from its bit fields (code 0: -9)."""
    e, m = (b >> 3) & 15, b & 7
    if e > 0:
        return e - 7
    return (int(m).bit_length() - 1) - 9 if m else -9


def edge_nvfp4_matrix(q: QMat, i: int, k: int, base: int) -> None:
    """Matrix i of an NVFP4 set: uniform random code bytes (all 16 E2M1 codes),
    each 16-element block's scale a random one of the 8 codes base .. base + 7,
    and a tensor scale that brings the weights to about 0.01-0.1 in size."""
    rows, cols = q.rows, q.cols
    q.codes[i] = uniform_bytes(key(k, TAG_EDGE, 0), rows * cols // 2).reshape(rows, cols // 2)
    off = uniform_bytes(key(k, TAG_EDGE, 1), rows * cols // 16) & 7
    q.scales[i] = (base + off).astype(np.uint8).reshape(rows, cols // 16)
    q.tensor_scale[i] = np.float32(0.01 * 2.0 ** -_e4m3_binade(base))


def edge_q4_1_matrix(q: QMat, i: int, k: int, regime: str) -> None:
    """Matrix i of a q4_1 set: uniform random code bytes and per-block {d, m}
    of a regime (fp16 values, rounded to nearest even by numpy):
      mixed          each block one of: d ~ 0.004, m ~ -7.5 d (the usual shape);
                     d = 0 with m = +-0.02 (constant blocks); d ~ 0.004 with
                     m > 0; d = m = 0;
      subnormal      d and m fp16 subnormals (random bit patterns), m of either sign;
      large          d in [100, 1000), m ~ -7.5 d (|d q + m| < 2^14);
      normal         d ~ 0.004 (0.5 .. 1.5), m ~ -7.5 d (0.8 .. 1.2);
      small_positive d ~ 1e-4, m = 0 (all weights >= 0)."""
    rows, cols = q.rows, q.cols
    nb = rows * cols // 32
    q.codes[i] = uniform_bytes(key(k, TAG_EDGE, 0), rows * cols // 2).reshape(rows, cols // 2)
    u = uniform_bytes(key(k, TAG_EDGE, 2), 4 * nb).reshape(4, nb).astype(np.float64) / 255.0
    sel = uniform_bytes(key(k, TAG_EDGE, 3), nb) & 3
    if regime == "mixed":
        d = 0.004 * (0.5 + u[0])
        m = np.where(sel == 0, -7.5 * d * (0.8 + 0.4 * u[1]),
                     np.where(sel == 1, 0.02 * (2 * u[1] - 1), np.where(sel == 2, 0.01 * u[1], 0.0)))
        d = np.where((sel == 1) | (sel == 3), 0.0, d)
        dm = np.stack([d.astype(np.float16).view(np.uint16), m.astype(np.float16).view(np.uint16)], -1)
    elif regime == "subnormal":
        db = uniform_bytes(key(k, TAG_EDGE, 4), 2 * nb).view(np.uint16) & 0x03FF
        sign = (sel.astype(np.uint16) & 1) << 15
        mb = (uniform_bytes(key(k, TAG_EDGE, 5), 2 * nb).view(np.uint16) & 0x03FF) | sign
        dm = np.stack([np.maximum(db, 1).astype(np.uint16), mb.astype(np.uint16)], -1)
    elif regime == "large":
        d = 100.0 + 900.0 * u[0]
        m = -7.5 * d * (0.9 + 0.2 * u[1])
        dm = np.stack([d.astype(np.float16).view(np.uint16), m.astype(np.float16).view(np.uint16)], -1)
    elif regime == "normal":
        d = 0.004 * (0.5 + u[0])
        m = -7.5 * d * (0.8 + 0.4 * u[1])
        dm = np.stack([d.astype(np.float16).view(np.uint16), m.astype(np.float16).view(np.uint16)], -1)
    elif regime == "small_positive":
        d = 1e-4 * (0.5 + u[0])
        dm = np.stack([d.astype(np.float16).view(np.uint16), np.zeros(nb, np.uint16)], -1)
    else:
        raise ValueError(regime)
    q.scales[i] = dm.reshape(rows, cols // 32, 2)


def make_edge_layer(fmt: str, seed: int = 0, E: int = 32, k: int = 2, n_shared: int = 1,
                    regimes: tuple | None = None) -> Layer:
    """A layer whose expert weights are patterned (N(0, 0.02) bf16 router, no
    bias).  NVFP4: routed expert e uses scale base E4M3_BASES[e % 32], the
    shared expert base 0x38.  q4_1: routed expert e uses regime
    regimes[e % len(regimes)] (default Q4_1_REGIMES), the shared expert
    'mixed'."""
    assert fmt in ("nvfp4", "q4_1")
    d, f = 2048, 512
    regimes = regimes or Q4_1_REGIMES
    router_w = normal_bf16(key(seed, TAG_ROUTER), 0.02, E * d).reshape(E, d)
    gate, up, down = alloc_qmat(fmt, E, f, d), alloc_qmat(fmt, E, f, d), alloc_qmat(fmt, E, d, f)

    def fill(qs, e, ek, sel):
        for j, q in enumerate(qs):
            kk = key(seed, TAG_EXPERT, ek, j)
            if fmt == "nvfp4":
                edge_nvfp4_matrix(q, e, kk, sel)
            else:
                edge_q4_1_matrix(q, e, kk, sel)

    for e in range(E):
        fill((gate, up, down), e, e, E4M3_BASES[e % 32] if fmt == "nvfp4" else regimes[e % len(regimes)])
    L = Layer(fmt, d, E, k, f, n_shared, 1.0, 1, router_w, None, gate, up, down,
              meta=dict(seed=seed, edge=True))
    if n_shared:
        L.sh_gate, L.sh_up, L.sh_down = alloc_qmat(fmt, 1, f, d), alloc_qmat(fmt, 1, f, d), alloc_qmat(fmt, 1, d, f)
        fill((L.sh_gate, L.sh_up, L.sh_down), 0, SHARED_ID, 0x38 if fmt == "nvfp4" else "mixed")
    return L


def make_edge_head(V: int, fmt: str, seed: int = 0) -> QMat:
    """Output-head matrix [V][2048] with patterned weights.  NVFP4: one tensor
    scale for the matrix, so row v's blocks use scale codes
    E4M3_BASES[v % 32] .. + 7 (rows differ in size by up to 2^17).  q4_1: row v
    in regime Q4_1_REGIMES[v % 5] (rows drawn as 1-row matrices)."""
    d = 2048
    q = alloc_qmat(fmt, 1, V, d)
    if fmt == "nvfp4":
        q.codes[0] = uniform_bytes(key(seed, TAG_EDGE, 10), V * d // 2).reshape(V, d // 2)
        off = uniform_bytes(key(seed, TAG_EDGE, 11), V * d // 16).reshape(V, d // 16) & 7
        base = np.array([E4M3_BASES[v % 32] for v in range(V)], np.uint8)[:, None]
        q.scales[0] = (base + off).astype(np.uint8)
        q.tensor_scale[0] = np.float32(1.0)
    else:
        row = alloc_qmat(fmt, 1, 1, d)
        for v in range(V):
            edge_q4_1_matrix(row, 0, key(seed, TAG_EDGE, 12, v), Q4_1_REGIMES[v % 5])
            q.codes[0, v] = row.codes[0, 0]
            q.scales[0, v] = row.scales[0, 0]
    return q


def make_x_rows(T: int, sigmas, xseed: int = 0, d: int = 2048) -> np.ndarray:
    """bf16 bits [T][d]: row t ~ bf16(fp32(N(0, sigma))) with sigma =
    sigmas[t % len(sigmas)] (sigma 0: an all-zero row)."""
    out = np.empty((T, d), np.uint16)
    for t in range(T):
        out[t] = normal_bf16(key(xseed, TAG_X, t + 1, 1), float(sigmas[t % len(sigmas)]), d)
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bits -> fp32 values (bit placement; exact)."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---- the five workloads -----------------------------------------------------------

CONFIGS = {
    # name: T, format, router skew, layers
    "decode_t4_q4_1": dict(T=4, fmt="q4_1", zipf=None, layers=1),
    "decode_t64_q4_1": dict(T=64, fmt="q4_1", zipf=None, layers=1),
    "decode_t256_nvfp4_zipf1.1": dict(T=256, fmt="nvfp4", zipf=1.1, layers=1),
    "prefill_t4096_bf16": dict(T=4096, fmt="bf16", zipf=None, layers=1),
    "stack47_decode_t32_q4_1_zipf0.8": dict(T=32, fmt="q4_1", zipf=0.8, layers=47),
}


# output-head workloads: name -> T, format, vocabulary
HEAD_CONFIGS = {
    "head_v151552_t1_q4_1": dict(T=1, fmt="q4_1", V=HEAD_VOCAB),
    "head_v151552_t4_q4_1": dict(T=4, fmt="q4_1", V=HEAD_VOCAB),
    "head_v151552_t8_q4_1": dict(T=8, fmt="q4_1", V=HEAD_VOCAB),
    "head_v151552_t16_q4_1": dict(T=16, fmt="q4_1", V=HEAD_VOCAB),
    "head_v151552_t32_q4_1": dict(T=32, fmt="q4_1", V=HEAD_VOCAB),
    "head_v151552_t64_q4_1": dict(T=64, fmt="q4_1", V=HEAD_VOCAB),
    "head_v151552_t4_nvfp4": dict(T=4, fmt="nvfp4", V=HEAD_VOCAB),
}


# decode-attention workloads: name -> sequences, cached positions, window, rotation
ATTN_CONFIGS = {
    "attn_full_b32_ctx8192": dict(B=32, ctx=8192, window=0, rope=False),
    "attn_swa_b32_ctx8192": dict(B=32, ctx=8192, window=ATTN_WINDOW, rope=True),
}


def make_workload(name: str, layers: int | None = None, workers: int = 1, progress=None):
    """(list of Layer, x) for a named workload.  Layer l of a stack is drawn
    from seed l; activations from seed 0.  `layers` truncates a stack.
    `workers` > 1 draws layers on threads (the C encoders release the GIL);
    `progress(l)` is called as layer l is ready.  The result does not depend
    on either."""
    c = CONFIGS[name]
    nl = c["layers"] if layers is None else layers

    def one(l):
        L = make_layer(seed=l, fmt=c["fmt"], zipf=c["zipf"])
        if progress is not None:
            progress(l)
        return L

    if workers > 1 and nl > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            Ls = list(ex.map(one, range(nl)))
    else:
        Ls = [one(l) for l in range(nl)]
    return Ls, make_x(c["T"])
