"""Pins for the oracle's output head (the 4-bit lm_head of the orcarouter.ai
review "Recursive Flint 40B-A2.5B", section "The quantisation recipe is the
most transferable part"): logits[t][v] = sum_k x[t][k] w[v][k].

What pins what:
  * the contraction: numpy's fp64 matmul of the decoded operands (a dropped
    term, a transposed operand or a wrong row fails it);
  * the row index: a one-hot token reads out one weight column, checked
    against bf16 bit placement for bf16 weights;
  * the decoders inside the head: matrices built by hand whose every weight is
    a closed form (q4_1 d*q + m with constant codes, NVFP4 E2M1 * E4M3 * ts),
    so that logits are that constant times the token sum;
  * sampled rows agree with the full evaluation; zero tokens give zero.
"""
import numpy as np
import pytest

import oracle
import synth


def head_matrix(fmt, V, d, seed=3):
    return synth.make_head(V, fmt, seed=seed, d=d)


@pytest.mark.parametrize("fmt,V,d", [("q4_1", 13, 64), ("nvfp4", 9, 64), ("bf16", 7, 64), ("q4_1", 3, 2048),
                                     ("nvfp4", 3, 2048)])
def test_head_matches_numpy_matmul_of_decoded_operands(fmt, V, d):
    q = head_matrix(fmt, V, d)
    x = synth.make_x(5, d, xseed=11)
    W = oracle.decode_matrix(q, 0).astype(np.float64)
    ref = synth.bf16_to_f32(x).astype(np.float64) @ W.T
    got = oracle.head_logits(q, x)
    assert got.shape == (5, V)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_one_hot_token_reads_one_bf16_weight_column():
    V, d = 11, 64
    q = head_matrix("bf16", V, d)
    x = np.zeros((d, d), np.uint16)
    x[np.arange(d), np.arange(d)] = 0x3F80  # bf16 1.0
    got = oracle.head_logits(q, x)  # [d][V]: token c selects column c
    W = synth.bf16_to_f32(q.codes[0]).astype(np.float64)  # [V][d], bit placement
    np.testing.assert_array_equal(got, W.T)


def test_q4_1_constant_codes_closed_form():
    V, d = 6, 2048
    q = synth.alloc_qmat("q4_1", 1, V, d)
    q.codes[:] = 0x55  # every nibble 5
    dv = np.array([0.25, -0.5, 0.125, 1.0, 0.0, 2.0], np.float16)
    mv = np.array([-1.0, 0.5, 0.0, -0.25, 3.0, 0.125], np.float16)
    q.scales[0, :, :, 0] = dv.view(np.uint16)[:, None]
    q.scales[0, :, :, 1] = mv.view(np.uint16)[:, None]
    x = synth.make_x(3, d, xseed=5)
    xs = synth.bf16_to_f32(x).astype(np.float64).sum(axis=1)
    w = 5 * dv.astype(np.float64) + mv.astype(np.float64)
    np.testing.assert_allclose(oracle.head_logits(q, x), xs[:, None] * w[None, :], rtol=1e-12, atol=1e-12)


def test_nvfp4_constant_codes_closed_form():
    V, d = 4, 2048
    q = synth.alloc_qmat("nvfp4", 1, V, d)
    q.codes[:] = 0x22  # E2M1 code 2 = 1.0 in both nibbles
    q.scales[0, :, :] = np.array([0x38, 0x40, 0x30, 0xB8], np.uint8)[:, None]  # 1, 2, 0.5, -1 in E4M3
    q.tensor_scale[0] = 0.75
    x = synth.make_x(2, d, xseed=6)
    xs = synth.bf16_to_f32(x).astype(np.float64).sum(axis=1)
    w = 0.75 * np.array([1.0, 2.0, 0.5, -1.0])
    np.testing.assert_allclose(oracle.head_logits(q, x), xs[:, None] * w[None, :], rtol=1e-12, atol=1e-12)


def test_sampled_rows_equal_the_full_evaluation_and_zero_tokens_give_zero():
    q = head_matrix("q4_1", 50, 64)
    x = synth.make_x(4, 64, xseed=2)
    full = oracle.head_logits(q, x)
    rows = np.array([49, 0, 17, 17, 3], np.int32)
    np.testing.assert_array_equal(oracle.head_logits(q, x, rows=rows), full[:, rows])
    z = oracle.head_logits(q, np.zeros((2, 64), np.uint16))
    assert np.all(z == 0)
    assert oracle.head_logits(q, np.zeros((0, 64), np.uint16)).shape == (0, 50)
