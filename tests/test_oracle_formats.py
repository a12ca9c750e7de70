"""Pins for the oracle's number-format decoders and the generator's encoders.

Each decoder is checked exhaustively against an independent definition:
numpy's IEEE binary16, the bit placement of bfloat16 inside binary32, torch's
float8_e4m3fn (OCP E4M3FN), and the E2M1 value list of the OCP microscaling
formats.  Encoder/decoder pairs are checked by round trips whose error bounds
follow from the formats alone, so a swapped nibble, a dropped min or a wrong
scale index fails them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def test_fp16_all_codes_match_numpy():
    codes = np.arange(65536, dtype=np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_value(int(c)) for c in codes])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.all(np.signbit(ref[~both_nan]) == np.signbit(got[~both_nan]))


def test_bf16_all_codes_match_fp32_bit_placement():
    codes = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):  # the NaN patterns widen to NaN
        ref = (codes << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_value(int(c)) for c in codes])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))


def test_e4m3_all_codes_match_torch_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(b) for b in range(256)])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    # special values of the OCP E4M3FN definition
    assert oracle.e4m3_value(0x00) == 0.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x7E) == 448.0
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert np.isnan(got).sum() == 2  # no infinities, two NaN codes


def test_e2m1_all_codes():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert abs(v) == mags[c & 7]
        assert (c >= 8) == (math.copysign(1.0, v) < 0)


@pytest.mark.parametrize("v,bits", [
    (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000),
    (1.0 + 2 ** -8, 0x3F80),            # halfway, even stays
    (1.0 + 3 * 2 ** -8, 0x3F82),        # halfway, rounds to even upward
    (1.0 + 2 ** -8 + 2 ** -30, 0x3F81),  # just above halfway
    (3.4e38, None),                     # near the top of the range: compare with torch
    (1e-40, None),                      # subnormal range
])
def test_bf16_rne_cases(v, bits):
    got = oracle.bf16_rne(v)
    if bits is None:
        ref = torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
        assert got == ref
    else:
        assert got == bits


def test_bf16_rne_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-38, rng.standard_normal(2000) * 1e30])
    v32 = v.astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_rne(float(x)) for x in v32], np.uint16)
    assert np.array_equal(got, ref)


def _q4_1_matrix(rows, cols, seed):
    w = synth.normal_f32(synth.key(seed, 99), 0.02, rows * cols).reshape(rows, cols)
    codes, dm = synth.encode_q4_1(w)
    q = synth.QMat("q4_1", 1, rows, cols, codes[None], dm[None])
    return w, q, codes, dm


def test_q4_1_round_trip_half_step():
    rows, cols = 16, 128
    w, q, codes, dm = _q4_1_matrix(rows, cols, 3)
    dec = oracle.decode_matrix(q, 0)
    d = dm[..., 0].view(np.float16).astype(np.float64)   # [rows][blocks]
    m = dm[..., 1].view(np.float16).astype(np.float64)
    err = np.abs(dec.astype(np.float64) - w.astype(np.float64)).reshape(rows, cols // 32, 32)
    # quantisation error <= half a step plus the fp16 rounding of the min
    bound = d[..., None] / 2 + np.abs(m[..., None] - w.reshape(rows, cols // 32, 32).min(-1, keepdims=True)) + 1e-9
    assert np.all(err <= bound)
    # nibble order: element 2i is the low nibble of byte i
    qn = np.empty((rows, cols), np.int64)
    qn[:, 0::2] = codes & 15
    qn[:, 1::2] = codes >> 4
    ref = (d.repeat(32, 1).astype(np.float32) * qn.astype(np.float32)) + m.repeat(32, 1).astype(np.float32)
    assert np.array_equal(dec, ref.astype(np.float32))


def test_q4_1_edge_blocks():
    cols = 32
    cases = [np.zeros(cols), np.full(cols, 0.5), np.linspace(-1, 1, cols), -np.linspace(1e-3, 2e-3, cols),
             np.array([65000.0] + [0.0] * (cols - 1)), np.full(cols, 1e-7)]
    for c in cases:
        w = c.astype(np.float32)[None]
        codes, dm = synth.encode_q4_1(w)
        q = synth.QMat("q4_1", 1, 1, cols, codes[None], dm[None])
        dec = oracle.decode_matrix(q, 0)[0].astype(np.float64)
        d = float(dm[0, 0, 0:1].view(np.float16)[0])
        mn = float(dm[0, 0, 1:2].view(np.float16)[0])
        assert np.all(np.abs(dec - c) <= d / 2 + abs(mn - c.min()) + 1e-12 + 1e-3 * abs(c).max())


def test_nvfp4_round_trip():
    rows, cols = 8, 64
    w = synth.normal_f32(synth.key(5, 99), 0.02, rows * cols).reshape(rows, cols)
    codes, sc, ts = synth.encode_nvfp4(w)
    q = synth.QMat("nvfp4", 1, rows, cols, codes[None], sc[None], np.array([ts], np.float32))
    dec = oracle.decode_matrix(q, 0).astype(np.float64)
    s = np.array([[oracle.e4m3_value(int(b)) for b in row] for row in sc]) * ts  # [rows][cols/16]
    # E2M1 spacing is at most 2 (between 4 and 6) in units of the block scale;
    # scale rounding to E4M3 can push a block amax up to 6*(1+1/16) -> clamp.
    err = np.abs(dec - w).reshape(rows, cols // 16, 16)
    assert np.all(err <= s[..., None] * 1.0 + 1e-12)
    # blockwise amax is represented within 1/8 relative (E4M3 has 3 mantissa bits)
    amax_b = np.abs(w).reshape(rows, cols // 16, 16).max(-1)
    assert np.all(np.abs(6 * s - amax_b) <= amax_b / 16 + 1e-12)
    assert np.linalg.norm(dec - w) / np.linalg.norm(w) < 0.12
    # code layout: element 2i is the low nibble of byte i, value E2M1 * E4M3 * ts
    qn = np.empty((rows, cols), np.int64)
    qn[:, 0::2] = codes & 15
    qn[:, 1::2] = codes >> 4
    e2 = np.array([oracle.e2m1_value(int(c)) for c in range(16)])[qn]
    ref = (e2 * s.repeat(16, 1) / ts).astype(np.float32) * np.float32(ts)
    assert np.array_equal(dec.astype(np.float32), ref)


def _scale_pos(k, C):
    """Storage position of block k's scales in a row of C blocks (the order the
    weight layout documents: k mod 16, then k // 16, where 16 divides C)."""
    G = 16 if C % 16 == 0 else C
    return (k % G) * (C // G) + k // G


def test_scale_order_is_a_permutation_pinned_at_2048_columns():
    pos = [_scale_pos(k, 64) for k in range(64)]
    assert sorted(pos) == list(range(64))
    assert pos[:3] == [0, 4, 8] and pos[16] == 1 and pos[17] == 5 and pos[63] == 63
    assert [_scale_pos(k, 16) for k in range(16)] == list(range(16))   # 512 columns: natural order
    assert [_scale_pos(k, 2) for k in range(2)] == [0, 1]


def test_q4_1_scales_of_2048_columns_follow_the_documented_order():
    rows, cols = 4, 2048
    w, q, codes, dm = _q4_1_matrix(rows, cols, 7)
    dec = oracle.decode_matrix(q, 0)
    pos = np.array([_scale_pos(k, cols // 32) for k in range(cols // 32)])
    d = dm[..., 0].view(np.float16).astype(np.float64)[:, pos]   # [rows][block]
    m = dm[..., 1].view(np.float16).astype(np.float64)[:, pos]
    qn = np.empty((rows, cols), np.int64)
    qn[:, 0::2] = codes & 15
    qn[:, 1::2] = codes >> 4
    ref = (d.repeat(32, 1).astype(np.float32) * qn.astype(np.float32)) + m.repeat(32, 1).astype(np.float32)
    assert np.array_equal(dec, ref.astype(np.float32))
    # the encoder stored each block's own scale there: the round trip is within half a step
    err = np.abs(dec.astype(np.float64) - w.astype(np.float64)).reshape(rows, cols // 32, 32)
    bound = d[..., None] / 2 + np.abs(m[..., None] - w.reshape(rows, cols // 32, 32).min(-1, keepdims=True)) + 1e-9
    assert np.all(err <= bound)


def test_nvfp4_scales_of_2048_columns_follow_the_documented_order():
    rows, cols = 4, 2048
    w = synth.normal_f32(synth.key(6, 99), 0.02, rows * cols).reshape(rows, cols)
    codes, sc, ts = synth.encode_nvfp4(w)
    q = synth.QMat("nvfp4", 1, rows, cols, codes[None], sc[None], np.array([ts], np.float32))
    dec = oracle.decode_matrix(q, 0)
    pos = np.array([_scale_pos(k, cols // 32) for k in range(cols // 32)])
    idx = (2 * pos[:, None] + np.arange(2)[None, :]).reshape(-1)   # 16-element block b -> storage byte
    s = np.array([[oracle.e4m3_value(int(v)) for v in row] for row in sc[:, idx]]) * ts
    qn = np.empty((rows, cols), np.int64)
    qn[:, 0::2] = codes & 15
    qn[:, 1::2] = codes >> 4
    e2 = np.array([oracle.e2m1_value(int(c)) for c in range(16)])[qn]
    ref = (e2 * s.repeat(16, 1) / ts).astype(np.float32) * np.float32(ts)
    assert np.array_equal(dec, ref)
    amax_b = np.abs(w).reshape(rows, cols // 16, 16).max(-1)
    assert np.all(np.abs(6 * s - amax_b) <= amax_b / 16 + 1e-12)


def test_nvfp4_encoder_ties_and_clamp():
    assert synth.lib().synth_f64_to_e2m1(0.25) == 0       # tie 0 / 0.5 -> even code 0
    assert synth.lib().synth_f64_to_e2m1(0.75) == 2       # tie 0.5 / 1 -> code 2 (1.0)
    assert synth.lib().synth_f64_to_e2m1(2.5) == 4        # tie 2 / 3 -> code 4 (2.0)
    assert synth.lib().synth_f64_to_e2m1(5.0) == 6        # tie 4 / 6 -> code 6 (4.0)
    assert synth.lib().synth_f64_to_e2m1(100.0) == 7      # clamp at 6
    assert synth.lib().synth_f64_to_e2m1(-1.6) == 8 + 3   # -1.5
    assert synth.lib().synth_f64_to_e4m3_sat(1000.0) == 0x7E
    assert synth.lib().synth_f64_to_e4m3_sat(2.0 ** -9) == 0x01
    for b in range(0x7F):  # every finite positive E4M3 value encodes to itself
        assert synth.lib().synth_f64_to_e4m3_sat(oracle.e4m3_value(b)) == b or oracle.e4m3_value(b) == 0


def test_bf16_weights_widen_exactly():
    rows, cols = 4, 32
    w = synth.normal_f32(synth.key(7, 99), 0.02, rows * cols).reshape(rows, cols)
    b = synth.encode_bf16(w)
    q = synth.QMat("bf16", 1, rows, cols, b[None])
    dec = oracle.decode_matrix(q, 0)
    assert np.array_equal(dec, synth.bf16_to_f32(b))
    assert np.max(np.abs(dec - w)) <= np.max(np.abs(w)) * 2 ** -8
