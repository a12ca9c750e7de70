"""The library's calls captured in a HIP graph and replayed: the layer forward
(at token counts with vector items only, with matrix-core tiles, and with the
chunked bucket build), a 3-layer stack, the output head (vector and
matrix-core kernels) and a decode-attention step (one split and several).

Each graph is replayed three times with eager work of the program (a torch
kernel on other memory) and synchronisations between the replays, and every
replay's output must equal the eager call's bit for bit: the kernels are
deterministic, and the calls write no memory with memset-type nodes.
"""
import numpy as np
import pytest
import torch

import quantized_expert_ffn_wave_amd as moe
import synth
from parity import say, x_to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def replay_matches(run, out, reps=3):
    """Capture run() (which writes `out`), then compare each replay with the
    eager result."""
    run()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    other = torch.ones(1 << 20, device="cuda")
    for r in range(reps):
        out.zero_()
        other.mul_(1.0001)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r} differs from the eager call"
    del g


@pytest.fixture(scope="module")
def layer():
    host = synth.make_layer(seed=3, fmt="q4_1")
    return host, moe.DeviceLayer(host, max_tokens=1024)


@pytest.mark.parametrize("T", [4, 64, 300])
def test_layer_forward_in_a_graph(layer, T):
    say(f"case graph layer T={T}")
    host, dl = layer
    x = x_to_dev(synth.make_x(T, xseed=T))
    y = torch.empty_like(x)
    ws = moe.alloc_workspace(dl.workspace_size(T))
    replay_matches(lambda: moe.layer_forward(dl, x, y, workspace=ws), y)


def test_stack_in_a_graph():
    say("case graph stack of 3 layers T=32")
    hosts = [synth.make_layer(seed=s, fmt="q4_1", zipf=0.8) for s in range(3)]
    dls = [moe.DeviceLayer(h, max_tokens=64) for h in hosts]
    x0 = x_to_dev(synth.make_x(32, xseed=5))
    x = x0.clone()
    ws = moe.alloc_workspace(moe.moe_stack_workspace_size([d.handle for d in dls], 32))

    def run():  # the stack updates x in place: start each run from the same input
        x.copy_(x0)
        moe.stack_forward(dls, x, workspace=ws)

    replay_matches(run, x)


@pytest.mark.parametrize("T", [4, 32])
def test_head_in_a_graph(T):
    say(f"case graph head T={T}")
    dm = moe.DeviceMatrix(synth.make_head(20000, "q4_1", seed=1))
    x = x_to_dev(synth.make_x(T, xseed=2))
    logits = torch.empty((T, 20000), dtype=torch.float32, device="cuda")
    replay_matches(lambda: moe.head_forward(dm, x, logits), logits)


@pytest.mark.parametrize("window,rope,cap", [(synth.ATTN_WINDOW, True, 1024), (0, False, 4096)])
def test_attention_in_a_graph(window, rope, cap):
    say(f"case graph attention window={window} cap={cap}")
    B = 8
    a = synth.make_attn(B, cap, seed=4)
    desc = moe.moe_attn_desc(window, int(rope), 10000.0, 1e-6)
    cache = moe.AttnCache(B, cap)
    cache.load(a["k_cache"], a["v_cache"])

    def dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).cuda().view(torch.bfloat16)

    q, k, v, qg, kg = dev(a["q"]), dev(a["k"]), dev(a["v"]), dev(a["q_gain"]), dev(a["k_gain"])
    sinks = torch.from_numpy(a["sinks"]).cuda()
    pos = torch.full((B,), cap - 1, dtype=torch.int32, device="cuda")
    out = torch.empty((B, synth.ATTN_HQ, synth.ATTN_D), dtype=torch.bfloat16, device="cuda")
    ws = moe.alloc_workspace(moe.attn_workspace_size(desc, B, cap))
    # appending the same token at the same position again leaves the cache as it was
    replay_matches(lambda: moe.attn_decode(desc, q, k, v, qg, kg, sinks, pos, cache, cap, out=out, workspace=ws), out)
