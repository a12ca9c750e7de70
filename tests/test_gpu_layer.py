"""GPU parity of one MoE layer (through the C ABI) against the CPU oracle.

Workloads: the decode layers of 4 and 64 tokens (q4_1, near-uniform routing),
256 tokens with NVFP4 weights and a Zipf(1.1) router bias, the 4096-token
bf16 prefill layer (outputs on a token sample), ragged token counts on both
sides of the small-bucket/large-bucket boundary, the largest accepted batch
(65536 tokens), reduced expert counts, top-k 1 and 8, no shared expert,
unnormalised weights, determinism and T=0.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_expert_ffn_wave_amd as moe
import synth
from parity import bits_of, check_layer, gpu_forward, say, x_to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


@pytest.fixture(scope="module")
def q4_layer():
    host = synth.make_layer(seed=0, fmt="q4_1")
    return host, moe.DeviceLayer(host, max_tokens=4096)


@pytest.fixture(scope="module")
def nvfp4_layer():
    host = synth.make_layer(seed=0, fmt="nvfp4", zipf=1.1)
    return host, moe.DeviceLayer(host, max_tokens=4096)


@pytest.fixture(scope="module")
def bf16_layer():
    host = synth.make_layer(seed=0, fmt="bf16")
    return host, moe.DeviceLayer(host, max_tokens=4096)


def test_decode_t4_q4_1(q4_layer):
    host, dl = q4_layer
    say("case decode_t4_q4_1")
    info = check_layer(host, synth.make_x(4), dl)
    say(f"  max row err {info['max_err']:.2e}")


def test_decode_t64_q4_1(q4_layer):
    host, dl = q4_layer
    say("case decode_t64_q4_1")
    info = check_layer(host, synth.make_x(64), dl)
    assert info["counts"].max() <= 8  # near-uniform load: small buckets
    say(f"  max row err {info['max_err']:.2e}, ties {info['ties']}")


@pytest.mark.parametrize("T", [1, 2, 3, 5, 7, 17, 63, 65, 100, 130])
def test_ragged_token_counts_q4_1(q4_layer, T):
    host, dl = q4_layer
    say(f"case q4_1 T={T}")
    check_layer(host, synth.make_x(T, xseed=100 + T), dl)


def test_decode_t256_nvfp4_zipf(nvfp4_layer):
    host, dl = nvfp4_layer
    say("case decode_t256_nvfp4_zipf1.1")
    info = check_layer(host, synth.make_x(256), dl)
    c = np.sort(info["counts"])[::-1]
    assert c[0] > 64 and (info["counts"] == 0).sum() > 100  # hot buckets, many empty experts
    say(f"  max row err {info['max_err']:.2e}, top buckets {c[:6].tolist()}")


@pytest.mark.parametrize("T", [1, 4, 33])
def test_nvfp4_small(nvfp4_layer, T):
    host, dl = nvfp4_layer
    say(f"case nvfp4 T={T}")
    check_layer(host, synth.make_x(T, xseed=200 + T), dl)


@pytest.mark.parametrize("T", [2, 64, 300])
def test_bf16_layer(bf16_layer, T):
    host, dl = bf16_layer
    say(f"case bf16 T={T}")
    check_layer(host, synth.make_x(T, xseed=300 + T), dl)


def test_prefill_t4096_bf16(bf16_layer):
    host, dl = bf16_layer
    say("case prefill_t4096_bf16 (outputs on 96 sampled tokens)")
    x = synth.make_x(4096)
    rng = np.random.default_rng(0)
    sample = np.concatenate([[0, 1, 4095], rng.choice(4096, 93, replace=False)])
    info = check_layer(host, x, dl, sample=sample)
    assert info["counts"].min() > 0 and 60 < info["counts"].mean() < 130
    say(f"  max row err {info['max_err']:.2e}")


def test_maximum_token_count_q4_1():
    """The largest batch a layer accepts (max_tokens = 65536): 16-bit token ids
    at their limit, 256 chunks in the bucket build, 128-token tiles only.  Routing
    is compared on every token, outputs on 64 sampled ones."""
    T = 65536
    host = synth.make_layer(seed=11, fmt="q4_1")
    dl = moe.DeviceLayer(host, max_tokens=T)
    say("case maximum token count q4_1 T=65536 (outputs on 64 sampled tokens)")
    x = synth.make_x(T, xseed=T)
    rng = np.random.default_rng(1)
    sample = np.concatenate([[0, 1, 32767, 65534, T - 1], rng.choice(T, 59, replace=False)])
    info = check_layer(host, x, dl, sample=sample)
    assert info["counts"].sum() == 6 * T and info["counts"].min() > 0
    say(f"  max row err {info['max_err']:.2e}")
    dl.close()


@pytest.mark.parametrize("E,k,n_shared,renorm,scale,fmt,T", [
    (16, 1, 1, 1, 1.0, "q4_1", 9),
    (16, 8, 1, 1, 1.0, "q4_1", 12),
    (32, 6, 0, 1, 1.0, "q4_1", 21),
    (32, 6, 1, 0, 2.5, "nvfp4", 19),
    (16, 6, 1, 1, 1.0, "bf16", 70),
    (32, 6, 1, 1, 1.0, "q4_1", 300),  # large-batch router and chunked buckets with fewer experts than waves
])
def test_layer_options(E, k, n_shared, renorm, scale, fmt, T):
    say(f"case options E={E} k={k} shared={n_shared} renorm={renorm} scale={scale} {fmt} T={T}")
    host = synth.make_layer(seed=7, fmt=fmt, E=E, k=k, n_shared=n_shared, renorm=renorm, shared_scale=scale,
                            zipf=0.5)
    check_layer(host, synth.make_x(T, xseed=400 + T), moe.DeviceLayer(host, max_tokens=T))


def test_small_and_large_bucket_boundary():
    """With 16 experts and top-6, token counts 8..14 give buckets of every size
    around the vector path's 4-token groups (one group, then two)."""
    host = synth.make_layer(seed=3, fmt="q4_1", E=16, k=6)
    dl = moe.DeviceLayer(host, max_tokens=64)
    seen = set()
    for T in range(8, 15):
        say(f"case boundary T={T}")
        info = check_layer(host, synth.make_x(T, xseed=500 + T), dl)
        seen |= set(info["counts"].tolist())
    assert {3, 4, 5, 6} <= seen


def test_deterministic_bits(q4_layer):
    host, dl = q4_layer
    say("case determinism T=64")
    x = synth.make_x(64, xseed=9)
    a = gpu_forward(dl, x, host.E, host.k)
    b = gpu_forward(dl, x, host.E, host.k)
    for n in ("topk_ids", "topk_w", "logits", "perm", "y_bits"):
        assert np.array_equal(a[n], b[n]), n


def test_zero_tokens_is_a_noop(q4_layer):
    host, dl = q4_layer
    say("case T=0")
    y = torch.full((1, 2048), 7.0, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((1, 2048), dtype=torch.bfloat16, device="cuda")
    ws = moe.alloc_workspace(dl.workspace_size(0))
    moe.moe_layer_forward(dl.handle, x.data_ptr(), 0, y.data_ptr(), None, ws.data_ptr(), ws.numel(),
                          moe.current_stream())
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


def test_forward_rejects_small_workspace_and_overlap(q4_layer):
    host, dl = q4_layer
    say("case argument errors")
    x = x_to_dev(synth.make_x(4))
    y = torch.empty_like(x)
    need = dl.workspace_size(4)
    ws = moe.alloc_workspace(need)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward(dl.handle, x.data_ptr(), 4, y.data_ptr(), None, ws.data_ptr(), need - 256,
                              moe.current_stream())
    assert e.value.status == moe.MOE_ERR_WORKSPACE
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward(dl.handle, x.data_ptr(), 4, x.data_ptr(), None, ws.data_ptr(), need,
                              moe.current_stream())
    assert e.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward(dl.handle, x.data_ptr(), 4097, y.data_ptr(), None, ws.data_ptr(), need,
                              moe.current_stream())
    assert e.value.status == moe.MOE_ERR_INVALID_ARG


def test_staged_forward_matches_plain_forward(q4_layer):
    """moe_layer_forward_staged records the stage events and computes the same bits."""
    host, dl = q4_layer
    say("case staged forward T=64")
    x = x_to_dev(synth.make_x(64, xseed=11))
    y0 = moe.layer_forward(dl, x)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(moe.N_STAGE_EVENTS)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    y1 = torch.empty_like(x)
    ws = moe.alloc_workspace(dl.workspace_size(64))
    moe.moe_layer_forward_staged(dl.handle, x.data_ptr(), 64, y1.data_ptr(), None, ws.data_ptr(), ws.numel(),
                                 moe.current_stream(), [e.cuda_event for e in ev])
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    t = [ev[i].elapsed_time(ev[i + 1]) for i in range(moe.N_STAGE_EVENTS - 1)]
    assert all(v >= 0 for v in t) and sum(t) > 0
    with pytest.raises(moe.MoeError):
        moe.moe_layer_forward_staged(dl.handle, x.data_ptr(), 64, y1.data_ptr(), None, ws.data_ptr(), ws.numel(),
                                     moe.current_stream(), [e.cuda_event for e in ev[:3]])


def test_matrix_core_bucket_boundary():
    """Buckets on both sides of the switch from 4-token vector groups to
    64-token matrix-core tiles: at 65 tokens in batches of up to 128 tokens
    (16 experts, top-8, 116..128 tokens), at 16 tokens in larger ones (64
    experts, top-6, 150..170 tokens)."""
    for E, k, Ts, lo, hi in ((16, 8, (116, 120, 124, 128), 64, 65), (64, 6, (150, 160, 170), 15, 16)):
        host = synth.make_layer(seed=5, fmt="q4_1", E=E, k=k)
        dl = moe.DeviceLayer(host, max_tokens=256)
        seen = set()
        for T in Ts:
            say(f"case matrix-core boundary E={E} k={k} T={T}")
            info = check_layer(host, synth.make_x(T, xseed=600 + T), dl)
            seen |= set(info["counts"].tolist())
        assert any(lo - 8 <= c <= lo for c in seen) and any(hi <= c <= hi + 8 for c in seen), sorted(seen)


def test_chunked_buckets_mixed(nvfp4_layer):
    """520 tokens: the 256-token chunked bucket build (last chunk ragged) with
    hot and mid-size matrix-core buckets and cold vector-path buckets (below 16
    tokens) in one batch."""
    host, dl = nvfp4_layer
    say("case chunked buckets nvfp4 zipf T=520")
    info = check_layer(host, synth.make_x(520, xseed=700), dl)
    c = info["counts"]
    assert c.max() >= 65 and ((c >= 16) & (c <= 64)).sum() > 5 and ((c > 0) & (c < 16)).sum() > 20
    say(f"  max row err {info['max_err']:.2e}")
