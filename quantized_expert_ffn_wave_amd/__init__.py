"""Python binding of libmoe_ffn.so, the gfx950 MoE-layer library.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI of include/moe_ffn.h.  torch is used for device
memory and the current stream.  The library must be built
(``python -m quantized_expert_ffn_wave_amd.build``); importing this package
without it raises ImportError -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_FFN_LIB") or os.path.join(_HERE, "libmoe_ffn.so")  # override: another build of the library

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE",
                4: "MOE_ERR_HIP"}
WFMT = {"bf16": 0, "q4_1": 1, "nvfp4": 2}
EXPORTED = ["moe_layer_create", "moe_layer_destroy", "moe_layer_workspace_size", "moe_desc_workspace_size",
            "moe_layer_forward", "moe_layer_forward_staged", "moe_layer_forward_noalloc",
            "moe_layer_forward_persistent", "moe_stack_workspace_size", "moe_stack_forward",
            "moe_stack_forward_persistent",
            "moe_head_forward", "moe_attn_workspace_size", "moe_attn_decode", "moe_stream_read", "moe_mfma_rate",
            "moe_read_pattern", "moe_release_cost",
            "moe_last_error",
            "moe_version"]
ATTN_HQ, ATTN_HK, ATTN_D = 32, 4, 128
HEAD_MAX_VOCAB = 1048576
N_STAGE_EVENTS = 7
STAGES = ["router", "topk", "bucket", "gate_up", "down", "combine"]

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m quantized_expert_ffn_wave_amd.build`")


class moe_layer_desc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_expert", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("d_shared", ctypes.c_int32),
                ("shared_scale", ctypes.c_float), ("renorm_topk", ctypes.c_int32), ("wfmt", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32)]


class moe_qmat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("tensor_scale", ctypes.c_void_p)]


class moe_layer_weights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("gate", moe_qmat), ("up", moe_qmat), ("down", moe_qmat),
                ("sh_gate", moe_qmat), ("sh_up", moe_qmat), ("sh_down", moe_qmat)]


class moe_attn_desc(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("rope", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rms_eps", ctypes.c_float)]


class moe_route_out(ctypes.Structure):
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("logits", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("x_in", ctypes.c_void_p), ("y_out", ctypes.c_void_p), ("inv_perm", ctypes.c_void_p)]


# torch is imported before the library is loaded so that one HIP runtime serves
# the process: torch brings its own libamdhip64 (soname libamdhip64.so.7), which
# then satisfies this library's dependency.  Loaded the other way round, the
# library would pull in the system runtime and torch a second one beside it,
# and the library's runtime then finds no device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_lib.moe_layer_create.argtypes = [ctypes.POINTER(moe_layer_desc), ctypes.POINTER(moe_layer_weights),
                                  ctypes.POINTER(_vp)]
_lib.moe_layer_create.restype = ctypes.c_int
_lib.moe_layer_destroy.argtypes = [_vp]
_lib.moe_layer_destroy.restype = None
_lib.moe_layer_workspace_size.argtypes = [_vp, _i32, ctypes.POINTER(_sz)]
_lib.moe_layer_workspace_size.restype = ctypes.c_int
_lib.moe_desc_workspace_size.argtypes = [ctypes.POINTER(moe_layer_desc), _i32, ctypes.POINTER(_sz)]
_lib.moe_desc_workspace_size.restype = ctypes.c_int
_lib.moe_layer_forward.argtypes = [_vp, _vp, _i32, _vp, ctypes.POINTER(moe_route_out), _vp, _sz, _vp]
_lib.moe_layer_forward.restype = ctypes.c_int
_lib.moe_layer_forward_staged.argtypes = [_vp, _vp, _i32, _vp, ctypes.POINTER(moe_route_out), _vp, _sz, _vp,
                                          ctypes.POINTER(_vp), _i32]
_lib.moe_layer_forward_staged.restype = ctypes.c_int
_lib.moe_layer_forward_noalloc.argtypes = [_vp, _vp, _i32, _vp, ctypes.POINTER(moe_route_out), _vp]
_lib.moe_layer_forward_noalloc.restype = ctypes.c_int
_lib.moe_stack_workspace_size.argtypes = [ctypes.POINTER(_vp), _i32, _i32, ctypes.POINTER(_sz)]
_lib.moe_stack_workspace_size.restype = ctypes.c_int
_lib.moe_stack_forward.argtypes = [ctypes.POINTER(_vp), _i32, _vp, _i32, ctypes.c_float,
                                   ctypes.POINTER(moe_route_out), _vp, _sz, _vp]
_lib.moe_stack_forward.restype = ctypes.c_int
_lib.moe_stack_forward_persistent.argtypes = _lib.moe_stack_forward.argtypes
_lib.moe_stack_forward_persistent.restype = ctypes.c_int
_lib.moe_layer_forward_persistent.argtypes = _lib.moe_layer_forward.argtypes
_lib.moe_layer_forward_persistent.restype = ctypes.c_int
_lib.moe_head_forward.argtypes = [_vp, _i32, ctypes.POINTER(moe_qmat), _i32, _i32, _i32, _vp, _vp]
_lib.moe_head_forward.restype = ctypes.c_int
_lib.moe_attn_workspace_size.argtypes = [ctypes.POINTER(moe_attn_desc), _i32, _i32, ctypes.POINTER(_sz)]
_lib.moe_attn_workspace_size.restype = ctypes.c_int
_lib.moe_attn_decode.argtypes = [ctypes.POINTER(moe_attn_desc), _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _i32, _vp, _vp, _sz, _vp]
_lib.moe_attn_decode.restype = ctypes.c_int
_lib.moe_stream_read.argtypes = [_vp, _sz, _vp, _i32, _vp]
_lib.moe_stream_read.restype = ctypes.c_int
_lib.moe_mfma_rate.argtypes = [_i32, _i32, _i32, _vp, _vp]
_lib.moe_mfma_rate.restype = ctypes.c_int
_lib.moe_read_pattern.argtypes = [_i32, _vp, _sz, _sz, _i32, _vp, _vp]
_lib.moe_read_pattern.restype = ctypes.c_int
_lib.moe_release_cost.argtypes = [_i32, _vp, _vp, _i32, _i32, _vp]
_lib.moe_release_cost.restype = ctypes.c_int
_lib.moe_last_error.restype = ctypes.c_char_p
_lib.moe_version.restype = ctypes.c_char_p


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.moe_last_error().decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def lib():
    return _lib


def version() -> str:
    return _lib.moe_version().decode()


def last_error() -> str:
    return _lib.moe_last_error().decode()


# ---- raw C-ABI calls (same names as include/moe_ffn.h) ------------------------------------

def moe_desc_workspace_size(desc: moe_layer_desc, T: int) -> int:
    n = _sz(0)
    _check(_lib.moe_desc_workspace_size(ctypes.byref(desc), T, ctypes.byref(n)), "moe_desc_workspace_size")
    return n.value


def moe_layer_create(desc: moe_layer_desc, weights: moe_layer_weights) -> int:
    h = _vp()
    _check(_lib.moe_layer_create(ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(h)), "moe_layer_create")
    return h.value


def moe_layer_destroy(handle: int) -> None:
    _lib.moe_layer_destroy(handle)


def moe_layer_workspace_size(handle: int, T: int) -> int:
    n = _sz(0)
    _check(_lib.moe_layer_workspace_size(handle, T, ctypes.byref(n)), "moe_layer_workspace_size")
    return n.value


def moe_layer_forward(handle: int, x_ptr: int, T: int, y_ptr: int, route: moe_route_out | None, ws_ptr: int,
                      ws_bytes: int, stream: int) -> None:
    _check(_lib.moe_layer_forward(handle, x_ptr, T, y_ptr, ctypes.byref(route) if route is not None else None,
                                  ws_ptr, ws_bytes, stream), "moe_layer_forward")


def moe_layer_forward_persistent(handle: int, x_ptr: int, T: int, y_ptr: int, route: moe_route_out | None,
                                 ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(_lib.moe_layer_forward_persistent(handle, x_ptr, T, y_ptr, ctypes.byref(route) if route is not None
                                             else None, ws_ptr, ws_bytes, stream), "moe_layer_forward_persistent")


PERSISTENT_MAX_T = 64


def moe_layer_forward_staged(handle: int, x_ptr: int, T: int, y_ptr: int, route: moe_route_out | None, ws_ptr: int,
                             ws_bytes: int, stream: int, events) -> None:
    """events: N_STAGE_EVENTS raw hipEvent_t handles (ints)."""
    arr = (_vp * len(events))(*events)
    _check(_lib.moe_layer_forward_staged(handle, x_ptr, T, y_ptr, ctypes.byref(route) if route is not None else None,
                                         ws_ptr, ws_bytes, stream, arr, len(events)), "moe_layer_forward_staged")


def moe_layer_forward_noalloc(handle: int, x_ptr: int, T: int, y_ptr: int, route: moe_route_out | None,
                              stream: int) -> None:
    _check(_lib.moe_layer_forward_noalloc(handle, x_ptr, T, y_ptr, ctypes.byref(route) if route is not None else None,
                                          stream), "moe_layer_forward_noalloc")


NOALLOC_MAX_WORKSPACE = 32 << 20


def moe_stack_workspace_size(handles, T: int) -> int:
    arr = (_vp * len(handles))(*handles)
    n = _sz(0)
    _check(_lib.moe_stack_workspace_size(arr, len(handles), T, ctypes.byref(n)), "moe_stack_workspace_size")
    return n.value


def moe_stack_forward(handles, x_ptr: int, T: int, eps: float, routes, ws_ptr: int, ws_bytes: int,
                      stream: int, persistent: bool = False) -> None:
    arr = (_vp * len(handles))(*handles)
    rarr = None
    if routes is not None:
        rarr = (moe_route_out * len(routes))(*routes)
    f = _lib.moe_stack_forward_persistent if persistent else _lib.moe_stack_forward
    _check(f(arr, len(handles), x_ptr, T, eps, rarr, ws_ptr, ws_bytes, stream),
           "moe_stack_forward_persistent" if persistent else "moe_stack_forward")



def moe_head_forward(x_ptr: int, T: int, w: moe_qmat, wfmt: int, vocab: int, d_model: int, logits_ptr: int,
                     stream: int) -> None:
    _check(_lib.moe_head_forward(x_ptr, T, ctypes.byref(w), wfmt, vocab, d_model, logits_ptr, stream),
           "moe_head_forward")


def moe_stream_read(src_ptr: int, nbytes: int, sink_ptr: int, grid: int, stream: int) -> None:
    _check(_lib.moe_stream_read(src_ptr, nbytes, sink_ptr, grid, stream), "moe_stream_read")


MFMA_KINDS = {0: ("v_mfma_f32_32x32x16_f16", 32768), 1: ("v_mfma_f32_32x32x16_bf16", 32768),
              2: ("v_mfma_f32_32x32x16_fp8_fp8", 32768), 3: ("v_mfma_scale_f32_32x32x64_f8f6f4 (fp4)", 131072)}


def moe_mfma_rate(kind: int, iters: int, grid: int, sink_ptr: int, stream: int) -> None:
    _check(_lib.moe_mfma_rate(kind, iters, grid, sink_ptr, stream), "moe_mfma_rate")


READ_PATTERNS = {0: ("contiguous 1 KB", 32), 1: ("32 rows x 32 B", 32), 2: ("32 rows x 64+64 B", 32),
                 3: ("4 rows x 256 B", 4), 4: ("8 rows x 128 B", 8)}  # name, rows per region


def moe_read_pattern(pattern: int, src_ptr: int, nbytes: int, row_bytes: int, grid: int, sink_ptr: int,
                     stream: int) -> None:
    _check(_lib.moe_read_pattern(pattern, src_ptr, nbytes, row_bytes, grid, sink_ptr, stream), "moe_read_pattern")


RELEASE_MODES = {0: "stores only", 1: "release + atomic", 2: "atomic only", 3: "release only",
                 4: "release + atomic + acquire"}


def moe_release_cost(mode: int, data_ptr: int, counters_ptr: int, grid: int, per_thread: int, stream: int) -> None:
    _check(_lib.moe_release_cost(mode, data_ptr, counters_ptr, grid, per_thread, stream), "moe_release_cost")


# ---- torch-level helpers -----------------------------------------------------------------

def make_desc(fmt: str, E: int = 256, k: int = 6, d: int = 2048, f: int = 512, n_shared: int = 1,
              shared_scale: float = 1.0, renorm: int = 1, max_tokens: int = 4096) -> moe_layer_desc:
    return moe_layer_desc(d, E, k, f, n_shared, f, shared_scale, renorm, WFMT[fmt], max_tokens)


def _to_dev(a: np.ndarray, device):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(device)


class DeviceLayer:
    """Weights of one layer copied to the device plus its library handle.

    `host` is any object with the attributes of a stored layer: fmt, E, k,
    n_shared, shared_scale, renorm, router_w (bf16 bits [E][d]), router_b
    (fp32 [E] or None) and gate/up/down/sh_gate/sh_up/sh_down, each with
    codes, scales, tensor_scale numpy arrays in the layouts of moe_ffn.h."""

    def __init__(self, host, device="cuda", max_tokens: int = 4096):
        self.keep = []
        self.fmt = host.fmt
        self.desc = make_desc(host.fmt, E=host.E, k=host.k, d=host.d, f=host.f, n_shared=host.n_shared,
                              shared_scale=host.shared_scale, renorm=host.renorm, max_tokens=max_tokens)
        w = moe_layer_weights()
        w.router_w = self._ptr(host.router_w, device)
        w.router_b = self._ptr(host.router_b, device) if host.router_b is not None else None
        for name in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
            q = getattr(host, name, None)
            if q is None:
                continue
            m = moe_qmat(self._ptr(q.codes, device),
                         self._ptr(q.scales, device) if q.scales is not None else None,
                         self._ptr(q.tensor_scale, device) if q.tensor_scale is not None else None)
            setattr(w, name, m)
        self.weights = w
        self.handle = moe_layer_create(self.desc, w)

    def _ptr(self, a, device):
        t = _to_dev(a, device)
        self.keep.append(t)
        return t.data_ptr()

    def workspace_size(self, T: int) -> int:
        return moe_layer_workspace_size(self.handle, T)

    def close(self):
        if self.handle:
            moe_layer_destroy(self.handle)
            self.handle = 0
            self.keep = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DeviceMatrix:
    """One stored matrix (matrix 0 of a host set with the attributes codes,
    scales, tensor_scale, fmt, rows, cols) copied to the device, with the
    moe_qmat that points at it."""

    def __init__(self, host, device="cuda"):
        self.fmt, self.rows, self.cols = host.fmt, host.rows, host.cols
        self.keep = []

        def ptr(a):
            if a is None:
                return None
            t = _to_dev(a, device)
            self.keep.append(t)
            return t.data_ptr()

        ts = host.tensor_scale[0:1] if host.tensor_scale is not None else None
        self.qmat = moe_qmat(ptr(host.codes[0]), ptr(host.scales[0] if host.scales is not None else None), ptr(ts))


def head_forward(m: DeviceMatrix, x, logits=None):
    """logits = x W^T for a bf16 torch tensor x [T][d] and a head matrix on the device."""
    import torch
    T = x.shape[0]
    if logits is None:
        logits = torch.empty((T, m.rows), dtype=torch.float32, device=x.device)
    moe_head_forward(x.data_ptr(), T, m.qmat, WFMT[m.fmt], m.rows, m.cols, logits.data_ptr(), current_stream())
    return logits


def attn_workspace_size(desc: moe_attn_desc, B: int, max_len: int) -> int:
    n = _sz(0)
    _check(_lib.moe_attn_workspace_size(ctypes.byref(desc), B, max_len, ctypes.byref(n)), "moe_attn_workspace_size")
    return n.value


def moe_attn_decode(desc: moe_attn_desc, B: int, max_len: int, q: int, k: int, v: int, q_gain: int, k_gain: int,
                    sinks, pos: int, k_cache: int, v_cache_t: int, cap: int, out: int, ws: int, ws_bytes: int,
                    stream: int) -> None:
    _check(_lib.moe_attn_decode(ctypes.byref(desc), B, max_len, q, k, v, q_gain, k_gain, sinks, pos, k_cache,
                                v_cache_t, cap, out, ws, ws_bytes, stream), "moe_attn_decode")


class AttnCache:
    """Device key/value cache of B sequences x cap positions in the library's
    layout (bf16; per (sequence, key-value head) a block of cap x 128):
    keys [cap/16][16 dimension groups][16 positions][8], values
    [cap/32][8 dimension groups][4][16 dimensions][8 positions]: within a
    32-position block, group g holds positions 4 g .. 4 g + 3 and 16 + 4 g ..
    16 + 4 g + 3."""

    def __init__(self, B: int, cap: int, device="cuda"):
        import torch
        self.B, self.cap = B, cap
        self.k = torch.zeros((B, ATTN_HK, cap // 16, ATTN_D // 8, 16, 8), dtype=torch.bfloat16, device=device)
        self.v_t = torch.zeros((B, ATTN_HK, cap // 32, ATTN_D // 16, 4, 16, 8), dtype=torch.bfloat16,
                               device=device)

    def load(self, k_plain: np.ndarray, v_plain: np.ndarray) -> None:
        """Fill from plain-layout bf16 bits [B][cap][4][128] (every position)."""
        import torch
        B, cap = self.B, self.cap
        kt = torch.from_numpy(np.ascontiguousarray(k_plain).view(np.int16)).view(torch.bfloat16)
        vt = torch.from_numpy(np.ascontiguousarray(v_plain).view(np.int16)).view(torch.bfloat16)
        # k[b][p][h][d], p = 16 pb + pi, d = 8 dg + di -> [b][h][pb][dg][pi][di]
        k6 = kt.reshape(B, cap // 16, 16, ATTN_HK, ATTN_D // 8, 8).permute(0, 3, 1, 4, 2, 5)
        self.k.copy_(k6.to(self.k.device))
        # v[b][p][h][d], p = 32 pb + 16 ph + 4 pg + ps, d = 16 dg + di -> [b][h][pb][dg][pg][di][ph][ps]
        v8 = vt.reshape(B, cap // 32, 2, 4, 4, ATTN_HK, ATTN_D // 16, 16).permute(0, 5, 1, 6, 3, 7, 2, 4)
        self.v_t.copy_(v8.reshape(self.v_t.shape).to(self.v_t.device))

    def plain(self):
        """(keys, values) as bf16 bits in the plain layout [B][cap][4][128]."""
        import torch
        B, cap = self.B, self.cap
        k = self.k.permute(0, 2, 4, 1, 3, 5).reshape(B, cap, ATTN_HK, ATTN_D)
        v8 = self.v_t.reshape(B, ATTN_HK, cap // 32, ATTN_D // 16, 4, 16, 2, 4)  # [b][h][pb][dg][pg][di][ph][ps]
        v = v8.permute(0, 2, 6, 4, 7, 1, 3, 5).reshape(B, cap, ATTN_HK, ATTN_D)
        k = k.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        v = v.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return k, v


def attn_decode(desc: moe_attn_desc, q, k, v, q_gain, k_gain, sinks, pos, cache: AttnCache, max_len: int,
                out=None, workspace=None):
    """One decode-attention step on torch device tensors (bf16 q [B][32][128],
    k, v [B][4][128], gains [128]; fp32 sinks [32] or None; int32 pos [B]).
    Appends k', v to the cache and returns out bf16 [B][32][128]."""
    import torch
    B = q.shape[0]
    if out is None:
        out = torch.empty((B, ATTN_HQ, ATTN_D), dtype=torch.bfloat16, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(attn_workspace_size(desc, B, max_len), device=q.device)
    moe_attn_decode(desc, B, max_len, q.data_ptr(), k.data_ptr(), v.data_ptr(), q_gain.data_ptr(),
                    k_gain.data_ptr(), None if sinks is None else sinks.data_ptr(), pos.data_ptr(),
                    cache.k.data_ptr(), cache.v_t.data_ptr(), cache.cap, out.data_ptr(), workspace.data_ptr(),
                    workspace.numel(), current_stream())
    return out


def alloc_workspace(nbytes: int, device="cuda"):
    """Caller-owned workspace (torch allocations are 256-byte aligned or better)."""
    import torch
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def route_buffers(T: int, k: int, E: int, device="cuda", d: int = 2048):
    """Device buffers for every moe_route_out field, and the struct pointing at them."""
    import torch
    b = dict(topk_ids=torch.empty((T, k), dtype=torch.int32, device=device),
             topk_w=torch.empty((T, k), dtype=torch.float32, device=device),
             logits=torch.empty((T, E), dtype=torch.float32, device=device),
             counts=torch.empty(E, dtype=torch.int32, device=device),
             offsets=torch.empty(E + 1, dtype=torch.int32, device=device),
             perm=torch.empty(max(T * k, 1), dtype=torch.int32, device=device),
             x_in=torch.empty((T, d), dtype=torch.bfloat16, device=device),
             y_out=torch.empty((T, d), dtype=torch.bfloat16, device=device),
             inv_perm=torch.empty(max(T * k, 1), dtype=torch.int32, device=device))
    r = moe_route_out(*[b[n].data_ptr() for n, _ in moe_route_out._fields_])
    return r, b


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def layer_forward(layer: DeviceLayer, x, y=None, route: moe_route_out | None = None, workspace=None,
                  persistent: bool = False):
    """y = MoE(x) for a bf16 torch tensor x [T][d] on the device (persistent:
    through moe_layer_forward_persistent)."""
    import torch
    T = x.shape[0]
    if y is None:
        y = torch.empty_like(x)
    nbytes = layer.workspace_size(T)
    if workspace is None:
        workspace = alloc_workspace(nbytes, x.device)
    f = moe_layer_forward_persistent if persistent else moe_layer_forward
    f(layer.handle, x.data_ptr(), T, y.data_ptr(), route, workspace.data_ptr(), workspace.numel(), current_stream())
    return y


def stack_forward(layers, x, eps: float = 1e-6, routes=None, workspace=None, persistent: bool = False):
    """In-place pre-norm residual stack over bf16 x [T][d]."""
    handles = [l.handle for l in layers]
    T = x.shape[0]
    nbytes = moe_stack_workspace_size(handles, T)
    if workspace is None:
        workspace = alloc_workspace(nbytes, x.device)
    moe_stack_forward(handles, x.data_ptr(), T, eps, routes, workspace.data_ptr(), workspace.numel(),
                      current_stream(), persistent=persistent)
    return x
