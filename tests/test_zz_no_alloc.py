"""The allocation-free layer forward (moe_layer_forward_noalloc) through the C
ABI against moe_layer_forward on the same inputs: bit-identical outputs and
routing copies, on two calls in a row (the second with fewer tokens, over the
scratch the first left behind), and its size limit."""
import numpy as np
import pytest
import torch

import quantized_expert_ffn_wave_amd as moe
import synth
from parity import bits_of, say, x_to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def run(dl, host, x, noalloc):
    T = x.shape[0]
    route, bufs = moe.route_buffers(T, host.k, host.E)
    y = torch.empty_like(x)
    if noalloc:
        moe.moe_layer_forward_noalloc(dl.handle, x.data_ptr(), T, y.data_ptr(), route, moe.current_stream())
    else:
        ws = moe.alloc_workspace(dl.workspace_size(T))
        moe.moe_layer_forward(dl.handle, x.data_ptr(), T, y.data_ptr(), route, ws.data_ptr(), ws.numel(),
                              moe.current_stream())
    torch.cuda.synchronize()
    out = {n: t.cpu().numpy() for n, t in bufs.items() if n not in ("x_in", "y_out")}
    out["y"] = bits_of(y)
    return out


@pytest.mark.parametrize("fmt,zipf,Ts", [("q4_1", None, (64, 5)), ("nvfp4", 1.1, (256, 17))])
def test_noalloc_matches_forward_twice(fmt, zipf, Ts):
    host = synth.make_layer(seed=2, fmt=fmt, zipf=zipf)
    dl = moe.DeviceLayer(host, max_tokens=4096)
    for i, T in enumerate(Ts):
        say(f"case noalloc {fmt} call {i + 1} T={T}")
        assert dl.workspace_size(T) <= moe.NOALLOC_MAX_WORKSPACE
        x = x_to_dev(synth.make_x(T, xseed=700 + T))
        ref = run(dl, host, x, noalloc=False)
        got = run(dl, host, x, noalloc=True)
        S = T * host.k
        for n in ("y", "topk_ids", "topk_w", "logits", "counts", "offsets"):
            assert np.array_equal(got[n], ref[n]), n
        for n in ("perm", "inv_perm"):
            assert np.array_equal(got[n][:S], ref[n][:S]), n
    dl.close()


def test_noalloc_rejects_forwards_beyond_its_scratch():
    host = synth.make_layer(seed=2, fmt="q4_1")
    dl = moe.DeviceLayer(host, max_tokens=4096)
    T = 4096
    say(f"case noalloc too large T={T}")
    assert dl.workspace_size(T) > moe.NOALLOC_MAX_WORKSPACE
    x = torch.zeros((T, 2048), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, 2048), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward_noalloc(dl.handle, x.data_ptr(), T, y.data_ptr(), None, moe.current_stream())
    assert e.value.status == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())  # nothing was enqueued
    dl.close()
