"""The persistent decode path (moe_layer_forward_persistent,
moe_stack_forward_persistent) through the C ABI: parity with the oracle and
bit-identity with the kernel chain of moe_layer_forward, on every format, the
token counts that pick each item size (1, up to 8, up to 64), reduced expert
counts and options, a stack, graph replays, and the 65-token rejection."""
import numpy as np
import pytest
import torch

import quantized_expert_ffn_wave_amd as moe
import synth
from parity import bits_of, check_layer, gpu_forward, say, x_to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

_L = {}


def layer(fmt, zipf=None, **kw):
    key = (fmt, zipf, tuple(sorted(kw.items())))
    if key not in _L:
        host = synth.make_layer(seed=12, fmt=fmt, zipf=zipf, **kw)
        _L[key] = (host, moe.DeviceLayer(host, max_tokens=128))
    return _L[key]


@pytest.mark.parametrize("fmt,zipf,T", [("q4_1", None, 1), ("q4_1", None, 4), ("q4_1", None, 8), ("q4_1", None, 9),
                                        ("q4_1", None, 33), ("q4_1", None, 64), ("nvfp4", 1.1, 5),
                                        ("nvfp4", 1.1, 64), ("bf16", None, 3), ("bf16", None, 40)])
def test_persistent_layer_parity_and_identity(fmt, zipf, T):
    host, dl = layer(fmt, zipf)
    x = synth.make_x(T, xseed=800 + T)
    say(f"case persistent {fmt} T={T}")
    info = check_layer(host, x, dl, persistent=True)
    ref = gpu_forward(dl, x, host.E, host.k)
    g = info["gpu"]
    for n in ("y_bits", "topk_ids", "topk_w", "logits", "counts", "offsets", "perm", "inv_perm"):
        assert np.array_equal(g[n], ref[n]), n
    say(f"  max row err {info['max_err']:.2e}, bit-identical to the kernel chain")


@pytest.mark.parametrize("E,k,n_shared,renorm,T", [(16, 8, 1, 1, 12), (32, 1, 0, 1, 7), (32, 6, 1, 0, 50)])
def test_persistent_layer_options(E, k, n_shared, renorm, T):
    host = synth.make_layer(seed=13, fmt="q4_1", E=E, k=k, n_shared=n_shared, renorm=renorm, zipf=0.5)
    dl = moe.DeviceLayer(host, max_tokens=T)
    x = synth.make_x(T, xseed=900 + T)
    say(f"case persistent options E={E} k={k} shared={n_shared} renorm={renorm} T={T}")
    info = check_layer(host, x, dl, persistent=True)
    ref = gpu_forward(dl, x, host.E, host.k)
    assert np.array_equal(info["gpu"]["y_bits"], ref["y_bits"])


def test_persistent_scaled_rows():
    host, dl = layer("q4_1")
    say("case persistent scaled rows T=30")
    check_layer(host, synth.make_x_rows(30, (1e-3, 1.0, 100.0, 0.0), xseed=5), dl, persistent=True)


def test_persistent_stack_matches_kernel_chain():
    from test_gpu_stack import run_stack, teacher_forced
    say("case persistent stack3 T=32 q4_1 zipf0.8")
    layers = [synth.make_layer(seed=40 + s, fmt="q4_1", zipf=0.8) for s in range(3)]
    x_bits = synth.make_x(32, xseed=41)
    out_ref, rec_ref = run_stack(layers, x_bits)
    dls = [moe.DeviceLayer(L, max_tokens=32) for L in layers]
    routes, bufs = zip(*[moe.route_buffers(32, L.k, L.E) for L in layers])
    x = x_to_dev(x_bits)
    moe.stack_forward(dls, x, routes=list(routes), persistent=True)
    torch.cuda.synchronize()
    out = bits_of(x)
    assert np.array_equal(out, out_ref)
    rec = []
    for b in bufs:
        rec.append(dict(topk_ids=b["topk_ids"].cpu().numpy(), topk_w=b["topk_w"].cpu().numpy(),
                        logits=b["logits"].cpu().numpy(), counts=b["counts"].cpu().numpy(),
                        offsets=b["offsets"].cpu().numpy(), perm=b["perm"].cpu().numpy(),
                        inv_perm=b["inv_perm"].cpu().numpy(), x_in=bits_of(b["x_in"]), y_out=bits_of(b["y_out"])))
    for r, q in zip(rec, rec_ref):
        assert np.array_equal(r["x_in"], q["x_in"]) and np.array_equal(r["y_out"], q["y_out"])
    teacher_forced(layers, x_bits, out, rec)


def test_persistent_graph_replays():
    host, dl = layer("q4_1")
    T = 16
    say("case persistent graph replays T=16")
    x = x_to_dev(synth.make_x(T, xseed=77))
    ws = moe.alloc_workspace(dl.workspace_size(T))
    y_eager = moe.layer_forward(dl, x, workspace=ws, persistent=True).clone()
    y = torch.empty_like(x)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_layer_forward_persistent(dl.handle, x.data_ptr(), T, y.data_ptr(), None, ws.data_ptr(), ws.numel(),
                                         moe.current_stream())
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16))


def test_persistent_rejects_batches_with_tiles():
    host, dl = layer("q4_1")
    say("case persistent T=65 rejected")
    x = torch.zeros((65, 2048), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    ws = moe.alloc_workspace(dl.workspace_size(65))
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward_persistent(dl.handle, x.data_ptr(), 65, y.data_ptr(), None, ws.data_ptr(),
                                         ws.numel(), moe.current_stream())
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED
