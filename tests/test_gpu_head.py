"""The output head (4-bit lm_head, orcarouter.ai review "Recursive Flint
40B-A2.5B", section "The quantisation recipe is the most transferable part")
on the GPU through the C ABI against the oracle.

Bar: per token, max_v |logit_gpu - logit_oracle| <= HEAD_TOL * max_v |logit_oracle|.
The kernel accumulates fp32 sums of exact fp16/bf16 products (q4_1 through its
1024-offset codes, whose block sums are formed at fp32 magnitudes of about
1024 * |sum x| and rounded to 2^-24 of that); the expected error is about
1e-5 of the row maximum, and a wrong row, token or K block moves a logit by
more than 1e-2 of it.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_expert_ffn_wave_amd as moe
import synth
from parity import say, x_to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

HEAD_TOL = 1e-3


def check(q, x_bits, rows=None):
    dm = moe.DeviceMatrix(q)
    x = x_to_dev(x_bits)
    got = moe.head_forward(dm, x)
    torch.cuda.synchronize()
    g = got.cpu().numpy().astype(np.float64)
    ref = oracle.head_logits(q, x_bits, rows=rows)
    if rows is not None:
        g = g[:, rows]
    assert np.isfinite(g).all()
    den = np.maximum(np.abs(ref).max(1), 1e-30)
    err = np.abs(g - ref).max(1) / den
    say(f"  max row-relative error {err.max():.2e}")
    assert err.max() <= HEAD_TOL, err
    return got


@pytest.mark.parametrize("fmt", ["q4_1", "nvfp4", "bf16"])
@pytest.mark.parametrize("V,T", [(1, 1), (3, 3), (63, 4), (64, 5), (65, 1), (1000, 17), (4097, 8)])
def test_head_small_vocab(fmt, V, T):
    say(f"case head fmt={fmt} V={V} T={T}")
    q = synth.make_head(V, fmt, seed=V)
    check(q, synth.make_x(T, xseed=T + 100))


@pytest.mark.parametrize("fmt,V,T", [("q4_1", synth.HEAD_VOCAB, 1), ("q4_1", synth.HEAD_VOCAB, 4),
                                     ("nvfp4", synth.HEAD_VOCAB, 4), ("bf16", synth.HEAD_VOCAB, 4),
                                     ("q4_1", 150001, 17), ("q4_1", synth.HEAD_VOCAB, 64)])
def test_head_full_vocab(fmt, V, T):
    """Full-size heads, every row against the oracle; T = 17 on a vocabulary of
    150001 rows has a ragged last row chunk and a token-group count that does
    not divide the grid (workgroups change token groups between items)."""
    say(f"case head fmt={fmt} V={V} T={T}")
    q = synth.make_head(V, fmt)
    check(q, synth.make_x(T, xseed=7))


def test_head_zero_tokens_writes_nothing():
    say("case head T=0")
    q = synth.make_head(100, "q4_1")
    dm = moe.DeviceMatrix(q)
    logits = torch.full((1, 100), 3.0, device="cuda")
    x = torch.zeros((1, 2048), dtype=torch.bfloat16, device="cuda")
    moe.moe_head_forward(x.data_ptr(), 0, dm.qmat, moe.WFMT["q4_1"], 100, 2048, logits.data_ptr(),
                         moe.current_stream())
    torch.cuda.synchronize()
    assert bool((logits == 3.0).all())


def test_head_leaves_logits_past_the_vocabulary_untouched():
    """A logits buffer wider than V x T: the kernel writes exactly T * V floats."""
    say("case head exact extent")
    V, T = 130, 5
    q = synth.make_head(V, "nvfp4", seed=9)
    dm = moe.DeviceMatrix(q)
    x = x_to_dev(synth.make_x(T, xseed=3))
    buf = torch.full((T * V + 64,), 7.0, device="cuda")
    moe.head_forward(dm, x, logits=buf[:T * V].view(T, V))
    torch.cuda.synchronize()
    assert bool((buf[T * V:] == 7.0).all())
    ref = oracle.head_logits(q, synth.make_x(T, xseed=3))
    g = buf[:T * V].view(T, V).cpu().numpy()
    assert (np.abs(g - ref).max(1) / np.abs(ref).max(1)).max() <= HEAD_TOL
