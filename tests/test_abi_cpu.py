"""The C-ABI library loads and exports every symbol include/moe_ffn.h declares;
host-side argument checks and workspace sizing (no GPU needed, no kernel runs)."""
import ctypes
import os
import re

import pytest

import quantized_expert_ffn_wave_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(moe.EXPORTED)
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_library_is_built_for_gfx950_only():
    blob = open(moe.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-+(gfx[0-9a-z]+)", blob))
    assert targets == {b"gfx950"}


def desc(**kw):
    d = moe.make_desc("q4_1")
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(n_experts=8), moe.MOE_ERR_INVALID_ARG),
    (dict(n_experts=257), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=9), moe.MOE_ERR_INVALID_ARG),
    (dict(n_shared=2), moe.MOE_ERR_INVALID_ARG),
    (dict(wfmt=7), moe.MOE_ERR_INVALID_ARG),
    (dict(max_tokens=0), moe.MOE_ERR_INVALID_ARG),
    (dict(d_shared=256), moe.MOE_ERR_INVALID_ARG),
    (dict(d_model=1024), moe.MOE_ERR_UNSUPPORTED),
    (dict(d_expert=256, d_shared=256), moe.MOE_ERR_UNSUPPORTED),
])
def test_bad_descriptors_are_rejected(kw, status):
    n = ctypes.c_size_t(0)
    st = moe.lib().moe_desc_workspace_size(ctypes.byref(desc(**kw)), 4, ctypes.byref(n))
    assert st == status
    assert moe.last_error()


def test_workspace_size_grows_with_tokens_and_rejects_bad_T():
    d = desc(max_tokens=4096)
    sizes = [moe.moe_desc_workspace_size(d, T) for T in (0, 1, 4, 64, 256, 4096)]
    assert all(b > a for a, b in zip(sizes, sizes[1:]))
    assert all(s % 256 == 0 for s in sizes)
    # the big terms: fp32 expert outputs and fp16 SwiGLU rows for S + T rows
    S = 64 * 6
    assert sizes[3] >= (S + 64) * (2048 * 4 + 512 * 2)
    n = ctypes.c_size_t(0)
    assert moe.lib().moe_desc_workspace_size(ctypes.byref(d), 4097, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    assert moe.lib().moe_desc_workspace_size(ctypes.byref(d), -1, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG


def fake_weights(align=256):
    base = 1 << 32
    q = moe.moe_qmat(base, base + align, base + 2 * align)
    return moe.moe_layer_weights(base, None, q, q, q, q, q, q)


def test_create_checks_pointers_before_the_device():
    out = ctypes.c_void_p()
    d = desc()
    w = fake_weights()
    w.router_w = None
    assert moe.lib().moe_layer_create(ctypes.byref(d), ctypes.byref(w), ctypes.byref(out)) == moe.MOE_ERR_INVALID_ARG
    w = fake_weights()
    w.gate = moe.moe_qmat((1 << 32) + 8, (1 << 32), None)  # codes not 16-byte aligned
    assert moe.lib().moe_layer_create(ctypes.byref(d), ctypes.byref(w), ctypes.byref(out)) == moe.MOE_ERR_INVALID_ARG
    assert "gate.codes" in moe.last_error()
    w = fake_weights()
    w.down = moe.moe_qmat(1 << 32, (1 << 32) + 4, None)  # q4_1 scales are read 16 bytes at a time
    assert moe.lib().moe_layer_create(ctypes.byref(d), ctypes.byref(w), ctypes.byref(out)) == moe.MOE_ERR_INVALID_ARG
    assert "down.scales" in moe.last_error()
    dn = moe.make_desc("nvfp4")
    w = fake_weights()
    w.up = moe.moe_qmat(1 << 32, 1 << 32, None)  # NVFP4 needs the per-matrix scale
    assert moe.lib().moe_layer_create(ctypes.byref(dn), ctypes.byref(w), ctypes.byref(out)) == moe.MOE_ERR_INVALID_ARG
    assert moe.lib().moe_layer_create(ctypes.byref(d), None, ctypes.byref(out)) == moe.MOE_ERR_INVALID_ARG
    assert moe.lib().moe_layer_create(None, ctypes.byref(fake_weights()), ctypes.byref(out)) == moe.MOE_ERR_INVALID_ARG


def test_create_without_a_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    out = ctypes.c_void_p()
    st = moe.lib().moe_layer_create(ctypes.byref(desc()), ctypes.byref(fake_weights()), ctypes.byref(out))
    assert st == moe.MOE_ERR_HIP
    assert out.value is None
    assert "hip" in moe.last_error().lower()


def test_forward_argument_errors_without_a_layer():
    lib = moe.lib()
    assert lib.moe_layer_forward(None, None, 4, None, None, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    n = ctypes.c_size_t(0)
    assert lib.moe_layer_workspace_size(None, 4, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    arr = (ctypes.c_void_p * 1)(None)
    assert lib.moe_stack_workspace_size(arr, 1, 4, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_stack_forward(None, 0, None, 4, 1e-6, None, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    lib.moe_layer_destroy(None)  # NULL-safe
    # the streaming-read helper checks its arguments before touching a device
    assert lib.moe_stream_read(None, 4096, 0x1000, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_stream_read(0x1008, 4096, 0x1000, 0, None) == moe.MOE_ERR_INVALID_ARG  # misaligned src
    assert lib.moe_stream_read(0x1000, 4100, 0x1000, 0, None) == moe.MOE_ERR_INVALID_ARG  # not 16 B multiple
    assert lib.moe_stream_read(0x1000, 4096, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_stream_read(0x1000, 4096, 0x1000, -1, None) == moe.MOE_ERR_INVALID_ARG
    assert moe.version().startswith("moe_ffn gfx950")


def test_head_argument_errors_before_the_device():
    """moe_head_forward checks every argument it can without a device; T = 0 is
    a no-op that succeeds once the matrix pointers check out."""
    lib = moe.lib()
    Q, BF, NV = moe.WFMT["q4_1"], moe.WFMT["bf16"], moe.WFMT["nvfp4"]
    good = moe.moe_qmat(0x1000, 0x2000, 0x3000)
    ref = ctypes.byref(good)
    X, L = 0x4000, 0x5000
    inv, uns = moe.MOE_ERR_INVALID_ARG, moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_head_forward(X, -1, ref, Q, 100, 2048, L, None) == inv
    assert lib.moe_head_forward(X, 65537, ref, Q, 100, 2048, L, None) == inv
    assert lib.moe_head_forward(X, 1, ref, Q, 0, 2048, L, None) == inv
    assert lib.moe_head_forward(X, 1, ref, Q, moe.HEAD_MAX_VOCAB + 1, 2048, L, None) == inv
    assert lib.moe_head_forward(X, 1, ref, 3, 100, 2048, L, None) == inv
    assert lib.moe_head_forward(X, 1, ref, Q, 100, 4096, L, None) == uns
    assert lib.moe_head_forward(X, 1, None, Q, 100, 2048, L, None) == inv
    assert lib.moe_head_forward(X, 1, ctypes.byref(moe.moe_qmat(0x1008, 0x2000, 0)), BF, 100, 2048, L, None) == inv
    assert lib.moe_head_forward(X, 1, ctypes.byref(moe.moe_qmat(0x1000, 0x2008, 0)), Q, 100, 2048, L, None) == inv
    assert lib.moe_head_forward(X, 1, ctypes.byref(moe.moe_qmat(0x1000, 0x2008, 0)), NV, 100, 2048, L, None) == inv
    assert "tensor_scale" in moe.last_error()
    assert lib.moe_head_forward(None, 1, ref, Q, 100, 2048, L, None) == inv
    assert lib.moe_head_forward(X + 8, 1, ref, Q, 100, 2048, L, None) == inv
    assert lib.moe_head_forward(X, 1, ref, Q, 100, 2048, None, None) == inv
    assert lib.moe_head_forward(X, 1, ref, Q, 100, 2048, L + 2, None) == inv
    assert lib.moe_head_forward(None, 0, ref, Q, 100, 2048, None, None) == moe.MOE_OK


def test_attention_argument_errors_before_the_device():
    """moe_attn_workspace_size / moe_attn_decode reject bad descriptors, sizes
    and pointers without touching a device; B = 0 is a no-op."""
    lib = moe.lib()
    inv, wsz = moe.MOE_ERR_INVALID_ARG, moe.MOE_ERR_WORKSPACE
    d = moe.moe_attn_desc(513, 1, 10000.0, 1e-6)
    n = ctypes.c_size_t(0)
    assert lib.moe_attn_workspace_size(ctypes.byref(d), 4, 1024, ctypes.byref(n)) == moe.MOE_OK
    need = n.value
    assert need > 0
    assert lib.moe_attn_workspace_size(None, 4, 1024, ctypes.byref(n)) == inv
    assert lib.moe_attn_workspace_size(ctypes.byref(d), 4, 1024, None) == inv
    for bad in (moe.moe_attn_desc(-1, 0, 1.0, 1e-6), moe.moe_attn_desc(0, 2, 1.0, 1e-6),
                moe.moe_attn_desc(0, 1, 0.0, 1e-6), moe.moe_attn_desc(0, 0, 1.0, -1.0)):
        assert lib.moe_attn_workspace_size(ctypes.byref(bad), 4, 1024, ctypes.byref(n)) == inv
    assert lib.moe_attn_workspace_size(ctypes.byref(d), -1, 1024, ctypes.byref(n)) == inv
    assert lib.moe_attn_workspace_size(ctypes.byref(d), 65536, 1024, ctypes.byref(n)) == inv
    assert lib.moe_attn_workspace_size(ctypes.byref(d), 4, 0, ctypes.byref(n)) == inv
    # more positions, more splits: the workspace grows
    big = ctypes.c_size_t(0)
    full = moe.moe_attn_desc(0, 0, 10000.0, 1e-6)
    assert lib.moe_attn_workspace_size(ctypes.byref(full), 4, 65536, ctypes.byref(big)) == moe.MOE_OK
    assert big.value > need

    P = [0x10000 + 0x1000 * i for i in range(12)]  # aligned fake device pointers

    def call(B=4, max_len=1024, cap=1024, ptrs=None, ws_bytes=need, desc=d):
        p = list(P) if ptrs is None else ptrs
        return lib.moe_attn_decode(ctypes.byref(desc), B, max_len, p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7],
                                   p[8], cap, p[9], p[10], ws_bytes, None)

    assert call(cap=1000) == inv            # not a multiple of 64
    assert call(cap=0) == inv
    assert call(max_len=2048) == inv        # beyond cap
    assert call(B=0) == moe.MOE_OK          # no-op, checked before the pointers
    for i in (0, 1, 2, 3, 4, 6, 7, 8, 9, 10):  # every pointer but sinks is required
        p = list(P)
        p[i] = 0
        assert call(ptrs=p) == inv, i
    p = list(P)
    p[0] += 8                                # q not 16-byte aligned
    assert call(ptrs=p) == inv
    p = list(P)
    p[10] += 16                              # workspace not 256-byte aligned
    assert call(ptrs=p) == inv
    p = list(P)
    p[5] += 2                                # sinks not 4-byte aligned
    assert call(ptrs=p) == inv
    assert call(ws_bytes=need - 1) == wsz


def test_one_hip_runtime_per_process():
    """Importing the binding alone leaves one libamdhip64 mapped (torch's), so
    that the library and torch share a runtime whatever is imported first."""
    import subprocess
    import sys
    code = ("import quantized_expert_ffn_wave_amd\n"
            "paths = set()\n"
            "for line in open('/proc/self/maps'):\n"
            "    p = line.split()[-1]\n"
            "    if 'libamdhip64' in p:\n"
            "        paths.add(os.path.realpath(p))\n"
            "print(len(paths), sorted(paths))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", "import os\n" + code], cwd=root, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    n = int(r.stdout.split()[0])
    assert n == 1, r.stdout


def test_measurement_helpers_check_arguments_before_the_device():
    """moe_read_pattern / moe_release_cost reject bad shapes and pointers
    without touching a device."""
    lib = moe.lib()
    inv = moe.MOE_ERR_INVALID_ARG
    src, sink = 0x100000, 0x2000
    rp = lambda p, nbytes, rb, grid=256, s=src, k=sink: lib.moe_read_pattern(p, s, nbytes, rb, grid, k, None)
    assert rp(5, 32 * 1024, 1024) == inv                # unknown pattern
    assert rp(0, 32 * 1024, 1000) == inv                # row_bytes not a multiple of 256
    assert rp(0, 31 * 1024, 1024) == inv                # not whole 32-row regions
    assert rp(3, 6 * 1024, 1024) == inv                 # not whole 4-row regions
    assert rp(4, 0, 1024) == inv
    assert rp(0, 32 * 1024, 1024, s=src + 8) == inv     # src not 16 B aligned
    assert rp(0, 32 * 1024, 1024, k=None) == inv
    assert rp(0, 32 * 1024, 1024, grid=0) == inv
    rc = lambda m, grid=64, pt=4, d=0x4000, c=0x8000: lib.moe_release_cost(m, d, c, grid, pt, None)
    assert rc(5) == inv and rc(-1) == inv
    assert rc(1, grid=0) == inv and rc(1, grid=65537) == inv
    assert rc(1, pt=0) == inv and rc(1, pt=65) == inv
    assert rc(1, d=None) == inv and rc(1, c=0x8002) == inv
    assert "counters" in moe.last_error()
