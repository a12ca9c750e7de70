"""The output head (4-bit lm_head, orcarouter.ai review "Recursive Flint
40B-A2.5B", section "The quantisation recipe is the most transferable part")
on the GPU through the C ABI against the oracle.

Bar: max over the case of |logit_gpu - logit_oracle| <= HEAD_TOL * RMS of the
case's oracle logits.  Up to 4 tokens the kernel multiplies exact fp16/bf16
products and accumulates in fp32 (errors near 1e-6 of the RMS).  Beyond 4
tokens it multiplies q4_1 weights decoded to fp16 (d q + m rounded once,
relative error <= 2^-11 per weight) on the matrix cores: with independent
roundings over 2048 terms that is about 1e-4 of the RMS per logit, and the
largest of ten million such errors stays below 1e-3 of it (an fp64 emulation
of that rounding reproduces the kernel's error to three digits).  A wrong row,
token or 32-element block moves a logit by more than 5e-2 of the RMS.
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

HEAD_TOL = 2e-3


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
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.abs(g - ref).max()) / rms
    say(f"  max error / rms {err:.2e}")
    assert err <= HEAD_TOL, err
    return got


_HEADS = {}


def head(V, fmt, seed=0):
    key = (V, fmt, seed)
    if key not in _HEADS:
        _HEADS.clear()  # one full-size head at a time in host memory
        _HEADS[key] = synth.make_head(V, fmt, seed=seed)
    return _HEADS[key]


# (V, T): token counts on every side of the pass sizes (1, 2, 4 and 8 token
# groups of 4 per pass; passes of 32 tokens beyond 32)
SMALL = [(1, 1), (3, 3), (63, 4), (64, 5), (65, 1), (63, 9), (1000, 17), (4097, 8), (65, 33), (3, 40), (200, 100)]


@pytest.mark.parametrize("fmt", ["q4_1", "nvfp4", "bf16"])
@pytest.mark.parametrize("V,T", SMALL)
def test_head_small_vocab(fmt, V, T):
    say(f"case head fmt={fmt} V={V} T={T}")
    check(synth.make_head(V, fmt, seed=V), synth.make_x(T, xseed=T + 100))


@pytest.mark.parametrize("fmt,V,T", [("q4_1", synth.HEAD_VOCAB, 1), ("q4_1", synth.HEAD_VOCAB, 4),
                                     ("q4_1", synth.HEAD_VOCAB, 8), ("q4_1", synth.HEAD_VOCAB, 16),
                                     ("q4_1", synth.HEAD_VOCAB, 32), ("q4_1", synth.HEAD_VOCAB, 33),
                                     ("q4_1", synth.HEAD_VOCAB, 64), ("q4_1", 150001, 17), ("q4_1", 150001, 40),
                                     ("nvfp4", synth.HEAD_VOCAB, 4), ("nvfp4", synth.HEAD_VOCAB, 32),
                                     ("bf16", synth.HEAD_VOCAB, 4), ("bf16", synth.HEAD_VOCAB, 20)])
def test_head_full_vocab(fmt, V, T):
    """Full-size heads, every row against the oracle.  A vocabulary of 150001
    rows ends in a ragged row chunk and leaves row chunks past the end in the
    item numbering; 33, 40 and 64 tokens take two passes (33: one token in the
    second)."""
    say(f"case head fmt={fmt} V={V} T={T}")
    check(head(V, fmt), synth.make_x(T, xseed=7))


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
    assert np.abs(g - ref).max() <= HEAD_TOL * np.sqrt(np.mean(ref * ref))
