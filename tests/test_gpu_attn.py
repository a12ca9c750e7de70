"""Decode attention (orcarouter.ai review "Recursive Flint 40B-A2.5B", section
"The architecture is an argument about memory bandwidth") on the GPU through
the C ABI against the oracle.

Checked per case:
  * the appended key k' and the prepared query q' (the workspace's first
    region, bf16 [B][32][128]) against the oracle's, within one bf16 step plus
    1e-5 (the kernel normalises and rotates in fp32, the oracle in fp64; both
    round to bf16, and values near a rounding boundary may land on either
    side);
  * the appended value bit for bit, and every other cache entry untouched;
  * the output against the oracle's attention over the GPU's own q' and cache
    (teacher-forced), element by element within
        2^-8 |ref| + 2^-7 * sum_j P_j |v_j| + 1e-6:
    the output is rounded to bf16 once (2^-9 relative) and the kernel
    multiplies bf16-rounded probabilities (2^-9 each, the same ones in the
    numerator and the denominator, so at most 2 * 2^-9 of sum_j P_j |v_j|);
    sum_j P_j |v_j| is the oracle's attention over |v|.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_expert_ffn_wave_amd as moe
import synth
from parity import say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

HQ, HK, D = synth.ATTN_HQ, synth.ATTN_HK, synth.ATTN_D


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f(b):
    return synth.bf16_to_f32(b).astype(np.float64)


def within_one_bf16_step(got, want):
    """|got - want| <= one bf16 step of want, plus 1e-5 for values near zero: a
    rotated element a cos - b sin can cancel to a tiny value, where the
    kernel's fp32 error (a few 2^-24 of the head's elements, which are of
    order 1) exceeds a step of the result."""
    g, w = f(got), f(want)
    step = np.abs(w) * 2.0 ** -7 + 1e-5
    return np.all(np.abs(g - w) <= step)


def run_case(B, cap, lens, window, rope, sinks=True, max_len=None, seed=0):
    lens = np.asarray(lens, np.int32)
    max_len = int(lens.max()) if max_len is None else max_len
    say(f"case attn B={B} cap={cap} lens={lens.tolist()[:6]} window={window} rope={rope} sinks={sinks} "
        f"max_len={max_len}")
    a = synth.make_attn(B, cap, seed=seed)
    pos = lens - 1
    desc = moe.moe_attn_desc(window, int(rope), 10000.0, 1e-6)
    cache = moe.AttnCache(B, cap)
    cache.load(a["k_cache"], a["v_cache"])
    sk = torch.from_numpy(a["sinks"]).cuda() if sinks else None
    ws = moe.alloc_workspace(moe.attn_workspace_size(desc, B, max_len))
    out = moe.attn_decode(desc, dev(a["q"]), dev(a["k"]), dev(a["v"]), dev(a["q_gain"]), dev(a["k_gain"]), sk,
                          torch.from_numpy(pos).cuda(), cache, max_len, workspace=ws)
    torch.cuda.synchronize()
    kc, vc = cache.plain()
    q_gpu = ws[:B * HQ * D * 2].view(torch.int16).cpu().numpy().view(np.uint16).reshape(B, HQ, D)
    q_ref, k_ref = oracle.attn_prep(a["q"], a["k"], a["q_gain"], a["k_gain"], pos, rope)
    assert within_one_bf16_step(q_gpu, q_ref)
    rows = np.arange(B)
    assert within_one_bf16_step(kc[rows, pos], k_ref)
    np.testing.assert_array_equal(vc[rows, pos], a["v"])
    untouched = np.ones((B, cap), bool)
    untouched[rows, pos] = False
    np.testing.assert_array_equal(kc[untouched], a["k_cache"][untouched])
    np.testing.assert_array_equal(vc[untouched], a["v_cache"][untouched])
    sinks_np = a["sinks"] if sinks else None
    ref = oracle.attn_decode(q_gpu, kc, vc, lens, window, sinks_np)
    mag = oracle.attn_decode(q_gpu, kc, vc & np.uint16(0x7FFF), lens, window, sinks_np)  # sum_j P_j |v_j|
    got = f(bits(out))
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -7 * mag + 1e-6
    say(f"  max err {err.max():.2e}, max err / bound {(err / bound).max():.3f}")
    assert np.isfinite(got).all()
    assert np.all(err <= bound)


def test_one_position_and_a_full_cache():
    run_case(2, 64, [1, 64], 0, False)


def test_window_edges_with_rotation():
    # exactly the window, one past it, and a window start that is not 64-aligned
    run_case(3, 640, [513, 514, 600], synth.ATTN_WINDOW, True)


def test_full_attention_ragged_lengths_without_sinks():
    run_case(4, 1024, [65, 127, 1000, 1024], 0, False, sinks=False)


def test_max_len_below_the_capacity():
    run_case(3, 1024, [700, 3, 64], 0, False, max_len=700)


def test_many_sequences_short_splits():
    # 64 sequences of up to 128 positions: the plan cuts 64-position splits
    rng = np.random.default_rng(5)
    run_case(64, 128, rng.integers(1, 129, 64), 0, True, seed=5)


def test_window_on_a_long_cache():
    run_case(2, 4096, [4096, 100], synth.ATTN_WINDOW, True, seed=2)


@pytest.mark.parametrize("window,rope", [(0, False), (synth.ATTN_WINDOW, True)])
def test_full_size_batch(window, rope):
    """The benchmark's shape: 32 sequences, 8192 positions each (full attention)
    or the 513-token window at position 8191."""
    run_case(32, 8192, np.full(32, 8192), window, rope, seed=7)


def test_positions_out_of_range_are_clamped():
    """pos outside [0, cap) is clamped into the cache, never written past it."""
    B, cap = 2, 64
    a = synth.make_attn(B, cap, seed=9)
    desc = moe.moe_attn_desc(0, 0, 10000.0, 1e-6)
    cache = moe.AttnCache(B, cap)
    cache.load(a["k_cache"], a["v_cache"])
    out = moe.attn_decode(desc, dev(a["q"]), dev(a["k"]), dev(a["v"]), dev(a["q_gain"]), dev(a["k_gain"]), None,
                          torch.tensor([-5, 1000], dtype=torch.int32, device="cuda"), cache, cap)
    torch.cuda.synchronize()
    kc, vc = cache.plain()
    np.testing.assert_array_equal(vc[[0, 1], [0, cap - 1]], a["v"])
    assert np.isfinite(f(bits(out))).all()


@pytest.mark.parametrize("window,lens", [(0, [5, 70, 130]), (synth.ATTN_WINDOW, [600, 514, 1000])])
def test_unwritten_cache_entries_never_reach_the_output(window, lens):
    """Every cache entry outside the attended positions holds a NaN; the output
    must still equal the oracle's (masked scores are selected away, masked
    values zeroed before their products)."""
    B, cap = len(lens), 1024
    lens = np.asarray(lens, np.int32)
    say(f"case attn NaN-filled cache window={window} lens={lens.tolist()}")
    a = synth.make_attn(B, cap, seed=11)
    kc, vc = a["k_cache"].copy(), a["v_cache"].copy()
    for b in range(B):
        lo = max(0, lens[b] - window) if window else 0
        keep = np.zeros(cap, bool)
        keep[lo:lens[b] - 1] = True  # the new token's slot is written by the call
        kc[b, ~keep] = 0x7FC0
        vc[b, ~keep] = 0x7FC0
    desc = moe.moe_attn_desc(window, int(window > 0), 10000.0, 1e-6)
    cache = moe.AttnCache(B, cap)
    cache.load(kc, vc)
    sk = torch.from_numpy(a["sinks"]).cuda()
    ws = moe.alloc_workspace(moe.attn_workspace_size(desc, B, cap))
    out = moe.attn_decode(desc, dev(a["q"]), dev(a["k"]), dev(a["v"]), dev(a["q_gain"]), dev(a["k_gain"]), sk,
                          torch.from_numpy(lens - 1).cuda(), cache, cap, workspace=ws)
    torch.cuda.synchronize()
    got = f(bits(out))
    assert np.isfinite(got).all()
    k2, v2 = cache.plain()
    q_gpu = ws[:B * HQ * D * 2].view(torch.int16).cpu().numpy().view(np.uint16).reshape(B, HQ, D)
    ref = oracle.attn_decode(q_gpu, k2, v2, lens, window, a["sinks"])
    mag = oracle.attn_decode(q_gpu, k2, v2 & np.uint16(0x7FFF), lens, window, a["sinks"])
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -7 * mag + 1e-6)
