"""Host checks of the patterned edge-case inputs (synth.make_edge_layer,
make_edge_head, make_x_rows): the stored codes cover what the GPU edge tests
claim to exercise.  No GPU."""
import numpy as np

import oracle
import synth


def nibbles(codes: np.ndarray) -> set:
    c = codes.ravel()
    return set(np.unique(c & 15).tolist()) | set(np.unique(c >> 4).tolist())


def test_nvfp4_edge_layer_uses_every_finite_scale_code_and_every_e2m1_code():
    L = synth.make_edge_layer("nvfp4", E=32, k=2, n_shared=1)
    codes = set()
    for q in (L.gate, L.up, L.down, L.sh_gate, L.sh_up, L.sh_down):
        codes |= set(np.unique(q.scales).tolist())
        assert nibbles(q.codes) == set(range(16))
        assert np.all(q.tensor_scale > 0)
    assert codes == set(range(256)) - {0x7F, 0xFF}
    # each routed expert holds the 8 codes from its base
    for e in (0, 15, 16, 31):
        b = synth.E4M3_BASES[e]
        assert set(np.unique(L.gate.scales[e]).tolist()) == set(range(b, b + 8))


def test_nvfp4_edge_weights_are_moderate_after_the_tensor_scale():
    L = synth.make_edge_layer("nvfp4", E=32, k=2, n_shared=0)
    for e in range(32):
        W = oracle.decode_matrix(L.down, e)
        a = np.abs(W[W != 0])
        if synth.E4M3_BASES[e] & 0x7F == 0:
            continue  # base 0: blocks of scale 0 and 2^-9 .. 7 * 2^-9
        assert 1e-4 < np.median(a) < 0.2, (e, np.median(a))


def test_q4_1_edge_regimes_have_their_properties():
    L = synth.make_edge_layer("q4_1", E=16, k=1, n_shared=0)
    f16 = lambda b: np.asarray(b, np.uint16).view(np.float16).astype(np.float64)
    for e in range(16):
        reg = synth.Q4_1_REGIMES[e % 5]
        dm = L.gate.scales[e].reshape(-1, 2)
        d, m = f16(dm[:, 0]), f16(dm[:, 1])
        assert nibbles(L.gate.codes[e]) == set(range(16))
        if reg == "mixed":
            assert (d == 0).any() and (m > 0).any() and (m < 0).any() and ((d == 0) & (m == 0)).any()
        elif reg == "subnormal":
            assert np.all((dm[:, 0] & 0x7C00) == 0) and np.all(dm[:, 0] & 0x3FF)
            assert np.all((dm[:, 1] & 0x7C00) == 0) and (m < 0).any() and (m > 0).any()
        elif reg == "large":
            assert d.min() >= 99 and np.all(np.maximum(np.abs(m), np.abs(15 * d + m)) < 2 ** 14)
        elif reg == "small_positive":
            assert np.all(m == 0) and np.all(d > 0)


def test_x_rows_take_their_scales():
    sig = (1e-3, 1.0, 0.0, 1e4)
    x = synth.bf16_to_f32(synth.make_x_rows(8, sig, xseed=1)).astype(np.float64)
    rms = np.sqrt(np.mean(x * x, axis=1))
    for t in range(8):
        s = sig[t % 4]
        if s == 0:
            assert not x[t].any()
        else:
            assert 0.9 * s < rms[t] < 1.1 * s
    assert not np.array_equal(x[1], x[5])  # distinct draws per row


def test_edge_head_rows():
    q = synth.make_edge_head(64, "nvfp4")
    for v in (0, 17, 63):
        b = synth.E4M3_BASES[v % 32]
        assert set(np.unique(q.scales[0, v]).tolist()) <= set(range(b, b + 8))
    q = synth.make_edge_head(10, "q4_1")
    dm = q.scales[0, 1].reshape(-1, 2)  # row 1: subnormal regime
    assert np.all((dm[:, 0] & 0x7C00) == 0)
