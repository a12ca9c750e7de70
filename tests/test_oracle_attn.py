"""Pins for the oracle's decode attention (the layout of the orcarouter.ai
review "Recursive Flint 40B-A2.5B", section "The architecture is an argument
about memory bandwidth": 32 query / 4 key-value heads of 128, a 513-token
sliding window or full attention, rotary embedding on the window layers only,
per-head QK RMSNorm, learned per-head sinks).

What pins what:
  * attention without a sink: torch's scaled_dot_product_attention in fp64
    with the key-value heads repeated for their 8 query heads (a transposed
    operand, a wrong head group or a wrong scale fails it);
  * the sink: one more logit in the denominator, so the output is the
    sink-free output times sum(e^s) / (sum(e^s) + e^z); with one cached
    position it is v * e^s / (e^s + e^z);
  * the window: the same as full attention over the last `window` positions;
  * RMSNorm: numpy's fp64 norm times the gain, within bf16 rounding;
  * rotation: identity at position 0 (bit for bit), the complex-number form
    (y_i + i y_{i+64}) = (x_i + i x_{i+64}) e^{i pos theta^(-i/64)}, and
    scores that depend only on the position difference.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

HQ, HK, D = synth.ATTN_HQ, synth.ATTN_HK, synth.ATTN_D


def f(b):
    return synth.bf16_to_f32(b).astype(np.float64)


def sdpa(q_bits, kc_bits, vc_bits, lens, lo=None):
    """torch fp64 attention of each sequence's token over positions lo .. len-1."""
    B = q_bits.shape[0]
    out = np.zeros((B, HQ, D))
    for b in range(B):
        a = 0 if lo is None else lo[b]
        q = torch.from_numpy(f(q_bits[b]))[:, None, :]                      # [HQ][1][D]
        k = torch.from_numpy(f(kc_bits[b, a:lens[b]])).permute(1, 0, 2)     # [HK][n][D]
        v = torch.from_numpy(f(vc_bits[b, a:lens[b]])).permute(1, 0, 2)
        k = k.repeat_interleave(HQ // HK, dim=0).contiguous()
        v = v.repeat_interleave(HQ // HK, dim=0).contiguous()
        out[b] = torch.nn.functional.scaled_dot_product_attention(q, k, v)[:, 0, :].numpy()
    return out


def test_attention_without_sink_matches_torch_sdpa():
    a = synth.make_attn(3, 40, seed=1)
    lens = np.array([40, 17, 1], np.int32)
    got = oracle.attn_decode(a["q"], a["k_cache"], a["v_cache"], lens, 0, None)
    np.testing.assert_allclose(got, sdpa(a["q"], a["k_cache"], a["v_cache"], lens), rtol=1e-11, atol=1e-12)


def test_sink_is_one_more_logit_in_the_denominator():
    a = synth.make_attn(2, 30, seed=2)
    lens = np.array([30, 9], np.int32)
    plain = oracle.attn_decode(a["q"], a["k_cache"], a["v_cache"], lens, 0, None)
    sunk = oracle.attn_decode(a["q"], a["k_cache"], a["v_cache"], lens, 0, a["sinks"])
    for b in range(2):
        q = f(a["q"][b])
        k = f(a["k_cache"][b, :lens[b]])                                       # [n][HK][D]
        s = np.einsum("hd,nhd->hn", q, np.repeat(k, HQ // HK, axis=1)) / np.sqrt(D)
        e = np.exp(s - s.max(1, keepdims=True))
        z = np.exp(a["sinks"].astype(np.float64) - s.max(1))
        factor = e.sum(1) / (e.sum(1) + z)
        np.testing.assert_allclose(sunk[b], plain[b] * factor[:, None], rtol=1e-11, atol=1e-13)


def test_single_position_closed_form():
    a = synth.make_attn(1, 4, seed=3)
    got = oracle.attn_decode(a["q"], a["k_cache"], a["v_cache"], np.array([1], np.int32), 0, a["sinks"])
    q, k, v = f(a["q"][0]), f(a["k_cache"][0, 0]), f(a["v_cache"][0, 0])
    for h in range(HQ):
        s = q[h] @ k[h // 8] / np.sqrt(D)
        w = 1.0 / (1.0 + np.exp(float(a["sinks"][h]) - s))
        np.testing.assert_allclose(got[0, h], w * v[h // 8], rtol=1e-12, atol=1e-14)


def test_window_is_full_attention_over_the_last_positions():
    a = synth.make_attn(3, 20, seed=4)
    lens = np.array([20, 5, 6], np.int32)
    W = 5
    got = oracle.attn_decode(a["q"], a["k_cache"], a["v_cache"], lens, W, None)
    ref = sdpa(a["q"], a["k_cache"], a["v_cache"], lens, lo=np.maximum(lens - W, 0))
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)
    # the window counts the current token: a length of exactly W is full attention
    full = oracle.attn_decode(a["q"], a["k_cache"], a["v_cache"], lens, 0, None)
    np.testing.assert_array_equal(got[1], full[1])


def _prep(a, pos, rope, B):
    return oracle.attn_prep(a["q"][:B], a["k"][:B], a["q_gain"], a["k_gain"], np.asarray(pos, np.int32), rope)


def test_rmsnorm_without_rotation():
    a = synth.make_attn(2, 1, seed=5)
    qo, ko = _prep(a, [7, 100], False, 2)
    for src, out, g in ((a["q"], qo, a["q_gain"]), (a["k"], ko, a["k_gain"])):
        x = f(src)
        exact = x / np.sqrt((x * x).mean(-1, keepdims=True) + 1e-6) * f(g)
        assert np.all(np.abs(f(out) - exact) <= np.abs(exact) * 2.0 ** -8 + 1e-30)


def test_rotation_is_identity_at_position_zero():
    a = synth.make_attn(1, 1, seed=6)
    q0, k0 = _prep(a, [0], True, 1)
    qn, kn = _prep(a, [0], False, 1)
    np.testing.assert_array_equal(q0, qn)
    np.testing.assert_array_equal(k0, kn)


@pytest.mark.parametrize("pos", [1, 37, 4096, 131071])
def test_rotation_complex_form(pos):
    a = synth.make_attn(1, 1, seed=7)
    qr, _ = _prep(a, [pos], True, 1)
    qn, _ = _prep(a, [pos], False, 1)
    x = f(qn[0])
    z = (x[:, :64] + 1j * x[:, 64:]) * np.exp(1j * pos * 10000.0 ** (-np.arange(64) / 64.0))
    exact = np.concatenate([z.real, z.imag], axis=1)
    # bf16 of the rotated fp64 value, against the rotation of the bf16 no-rotation value
    assert np.abs(f(qr[0]) - exact).max() <= 2.0 ** -7 * np.abs(exact).max()


def test_scores_depend_only_on_the_position_difference():
    a = synth.make_attn(1, 1, seed=8)
    qa, _ = _prep(a, [50], True, 1)
    _, ka = _prep(a, [20], True, 1)
    qb, _ = _prep(a, [1050], True, 1)
    _, kb = _prep(a, [1020], True, 1)
    sa = np.einsum("hd,hd->h", f(qa[0])[:4], f(ka[0]))
    sb = np.einsum("hd,hd->h", f(qb[0])[:4], f(kb[0]))
    np.testing.assert_allclose(sa, sb, atol=0.05 * np.abs(sa).max())
