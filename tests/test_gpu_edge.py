"""GPU parity on edge-case weights and token rows, through the C ABI, against the oracle.

The stored formats are the review's ("Recursive Flint 40B-A2.5B", section
"What actually shipped": the NVFP4 and Int4 (q4_1) GGUF bullets).  Every test
compares the HIP path with the oracle under the rules of parity.py:
  * NVFP4 weights whose 16-element blocks take every finite E4M3 scale code of
    both signs and whose codes take all 16 E2M1 values, on the vector path, on
    64-token tiles and on 128-token tiles;
  * q4_1 blocks with d = 0, fp16-subnormal d and m, positive m and large d; each
    expert holds one regime and each token is routed to one expert with no
    shared expert, so that a token's output row isolates one regime;
  * token rows scaled by 1e-5 .. 1e4, and all-zero rows (whose output must be
    exactly zero);
  * the output head on the same weight patterns: every logit within a
    forward-error bound of the oracle's, 1e-3 * sum_k |x_k w_vk|;
  * RMSNorm's epsilon inside the square root, in the stack, on token rows whose
    mean square is about eps.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_expert_ffn_wave_amd as moe
import synth
from parity import check_layer, say, x_to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

# token-row scales (sigma of the N(0, sigma) draw; 0 = an all-zero row)
SIGMAS = (1e-3, 1e-2, 1.0, 100.0, 0.0, 1e-5, 1e4)

_CACHE = {}


def edge_layer(fmt, **kw):
    key = (fmt, tuple(sorted(kw.items())))
    if key not in _CACHE:
        host = synth.make_edge_layer(fmt, seed=21, **kw)
        _CACHE[key] = (host, moe.DeviceLayer(host, max_tokens=1024))
    return _CACHE[key]


@pytest.mark.parametrize("T", [128, 256, 1024])
def test_nvfp4_every_scale_code(T):
    """E = 32 routed experts (expert e: scale codes E4M3_BASES[e] .. + 7, so the
    32 experts hold all 254 finite codes) + a shared one, top-2.  T = 128: every
    routed bucket on the vector path; 256: vector and 64-token tiles; 1024:
    128-token tiles only."""
    host, dl = edge_layer("nvfp4", E=32, k=2, n_shared=1)
    say(f"case nvfp4 every scale code T={T}")
    info = check_layer(host, synth.make_x_rows(T, SIGMAS, xseed=T), dl)
    c = info["counts"]
    assert (c > 0).all(), c  # every expert, hence every scale code, took part
    if T == 128:
        assert c.max() < 65
    if T == 256:
        assert c.max() >= 16 and c.min() < 16
    if T == 1024:
        assert c.min() >= 16
    say(f"  max row err {info['max_err']:.2e}, buckets {c.min()}..{c.max()}")


@pytest.mark.parametrize("T", [64, 256, 1024])
def test_q4_1_edge_blocks_isolated(T):
    """16 routed experts, expert e in regime Q4_1_REGIMES[e % 5], top-1 and no
    shared expert: each output row is one expert's on one scaled token row."""
    host, dl = edge_layer("q4_1", E=16, k=1, n_shared=0)
    say(f"case q4_1 edge blocks isolated T={T}")
    info = check_layer(host, synth.make_x_rows(T, SIGMAS, xseed=50 + T), dl)
    c = info["counts"]
    regimes = {synth.Q4_1_REGIMES[e % 5] for e in range(16) if c[e] > 0}
    assert regimes == set(synth.Q4_1_REGIMES), regimes
    if T == 1024:
        assert c[c > 0].min() >= 16
    say(f"  max row err {info['max_err']:.2e}, touched {(c > 0).sum()}")


@pytest.mark.parametrize("T", [40, 128])
def test_q4_1_mixed_blocks_with_shared(T):
    """Every expert, the shared one included, in the 'mixed' regime (d = 0 blocks,
    positive and negative m, zero blocks), top-6 of 32."""
    host, dl = edge_layer("q4_1", E=32, k=6, n_shared=1, regimes=("mixed",))
    say(f"case q4_1 mixed blocks shared T={T}")
    info = check_layer(host, synth.make_x_rows(T, SIGMAS, xseed=80 + T), dl)
    say(f"  max row err {info['max_err']:.2e}")


@pytest.mark.parametrize("fmt,T,zipf", [("q4_1", 64, None), ("q4_1", 300, None), ("nvfp4", 256, 1.1),
                                        ("bf16", 300, None)])
def test_scaled_rows_standard_layers(fmt, T, zipf):
    """The standard synthetic layers (N(0, 0.02) weights) on scaled and zero rows."""
    host = synth.make_layer(seed=4, fmt=fmt, zipf=zipf)
    say(f"case scaled rows {fmt} T={T}")
    info = check_layer(host, synth.make_x_rows(T, SIGMAS, xseed=90 + T), moe.DeviceLayer(host, max_tokens=T))
    say(f"  max row err {info['max_err']:.2e}")


def test_zero_rows_give_zero_output():
    host, dl = edge_layer("nvfp4", E=32, k=2, n_shared=1)
    say("case all-zero rows")
    x = np.zeros((8, 2048), np.uint16)
    y = moe.layer_forward(dl, x_to_dev(x))
    torch.cuda.synchronize()
    assert not bool(y.view(torch.int16).abs().sum())


HEAD_BOUND = 1e-3


@pytest.mark.parametrize("fmt", ["nvfp4", "q4_1"])
@pytest.mark.parametrize("T", [4, 16, 40])
def test_head_edge_rows(fmt, T):
    """Head rows in the patterned formats (NVFP4: row v's scale codes from
    E4M3_BASES[v % 32], one tensor scale, so rows differ in size by up to 2^17;
    q4_1: row v in regime v % 5) against scaled and zero token rows.  Each logit
    must be within 1e-3 * sum_k |x_k w_vk| of the oracle's: fp16 rounding of a
    q4_1 weight (2^-11 of it) and fp32 accumulation over 2048 terms stay below
    that, while a wrong scale code, block or row moves a logit by a large part
    of its own size.  T = 4: the vector kernel; 16: one matrix-core pass; 40:
    two passes of 32."""
    V = 640
    q = synth.make_edge_head(V, fmt, seed=T)
    x_bits = synth.make_x_rows(T, SIGMAS, xseed=120 + T)
    say(f"case head edge {fmt} V={V} T={T}")
    got = moe.head_forward(moe.DeviceMatrix(q), x_to_dev(x_bits))
    torch.cuda.synchronize()
    g = got.cpu().numpy().astype(np.float64)
    ref = oracle.head_logits(q, x_bits)
    W = oracle.decode_matrix(q, 0).astype(np.float64)
    B = np.abs(synth.bf16_to_f32(x_bits).astype(np.float64)) @ np.abs(W).T
    assert np.isfinite(g).all()
    err = np.abs(g - ref)
    assert np.all(err <= HEAD_BOUND * B), float((err / np.maximum(B, 1e-300)).max())
    zero = np.array([SIGMAS[t % len(SIGMAS)] == 0.0 for t in range(T)])
    assert not g[zero].any()
    say(f"  max error / bound {(err / np.maximum(B, 1e-300)).max() / HEAD_BOUND:.2e}")


def test_stack_rmsnorm_eps_inside_the_root():
    """Rows of RMS 1e-3 (mean square 1e-6 = eps): the stack's first layer input
    must be bf16(r / sqrt(mean(r^2) + eps)), about r / (1.41e-3); eps outside the
    root would give about r / 1e-3.  Checked teacher-forced on every layer and
    free-running, with the stack tests' rules."""
    from test_gpu_stack import free_running, run_stack, teacher_forced
    say("case stack rmsnorm eps T=16 rows of RMS 1e-3")
    layers = [synth.make_layer(seed=30 + s, fmt="q4_1") for s in range(2)]
    x = synth.make_x_rows(16, (1e-3,), xseed=33)
    out, rec = run_stack(layers, x)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    x0 = synth.bf16_to_f32(rec[0]["x_in"]).astype(np.float64)
    ratio = np.sqrt(np.mean(x0 * x0, axis=1)) / np.sqrt(np.mean(xf * xf, axis=1))
    expect = 1.0 / np.sqrt(np.mean(xf * xf, axis=1) + 1e-6)
    assert np.all(np.abs(ratio / expect - 1) < 1e-2), ratio / expect
    teacher_forced(layers, x, out, rec)
    free_running(layers, x, out, rec, sample=np.arange(16))
