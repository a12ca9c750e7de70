"""GPU parity of the pre-norm residual stack (moe_stack_forward) against the oracle.

Two checks per stack:
  * teacher-forced, layer by layer: the oracle runs each layer on the GPU's
    own bf16 layer input (route.x_in) and must agree with the GPU's routing and
    bf16 layer output (route.y_out) under the single-layer rules; the GPU's
    next input must be bf16(RMSNorm(r)) of the residual rebuilt from its
    outputs;
  * free-running: the oracle's whole stack on a token sample must match the
    GPU's final bf16 output, except tokens whose routing took the other valid
    choice at a near-tie (reported, and covered by the teacher-forced check).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_expert_ffn_wave_amd as moe
import synth
from parity import EPS, OUT_TOL, bits_of, check_routing, row_rel_err, say, x_to_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def run_stack(layers, x_bits, eps=1e-6):
    T = x_bits.shape[0]
    dls = [moe.DeviceLayer(L, max_tokens=T) for L in layers]
    routes, bufs = [], []
    for L in layers:
        r, b = moe.route_buffers(T, L.k, L.E)
        routes.append(r)
        bufs.append(b)
    x = x_to_dev(x_bits)
    moe.stack_forward(dls, x, eps=eps, routes=routes)
    torch.cuda.synchronize()
    rec = []
    for b in bufs:
        rec.append(dict(topk_ids=b["topk_ids"].cpu().numpy(), topk_w=b["topk_w"].cpu().numpy(),
                        logits=b["logits"].cpu().numpy(), counts=b["counts"].cpu().numpy(),
                        offsets=b["offsets"].cpu().numpy(), perm=b["perm"].cpu().numpy()[:T * layers[0].k],
                        inv_perm=b["inv_perm"].cpu().numpy()[:T * layers[0].k],
                        x_in=bits_of(b["x_in"]), y_out=bits_of(b["y_out"])))
    for d in dls:
        d.close()
    return bits_of(x), rec


def teacher_forced(layers, x_bits, out_bits, rec, eps=1e-6, layer_ids=None, threads=0):
    T, d = x_bits.shape
    r = synth.bf16_to_f32(x_bits).astype(np.float32)
    worst = 0.0
    for l, L in enumerate(layers):
        g = rec[l]
        # the layer input is bf16(RMSNorm(r)) of the residual so far
        xn_ref = np.stack([oracle.rmsnorm_bf16(row.astype(np.float64), eps) for row in r])
        a = synth.bf16_to_f32(g["x_in"]).astype(np.float64)
        b = synth.bf16_to_f32(xn_ref).astype(np.float64)
        assert np.all(np.abs(a - b) <= np.abs(b) * 2 ** -7 + 1e-30), l
        if layer_ids is None or l in layer_ids:
            o = oracle.route(L, g["x_in"], threads=threads)
            o["renorm"] = L.renorm
            check_routing(g, o, L.E, L.k)
            ref = oracle.layer_forward(L, g["x_in"], forced_ids=g["topk_ids"], threads=threads)
            err = row_rel_err(synth.bf16_to_f32(g["y_out"]).astype(np.float64), ref["out"])
            assert err.max() <= OUT_TOL, (l, err.max())
            worst = max(worst, float(err.max()))
        r = r + synth.bf16_to_f32(g["y_out"])  # fp32 residual, as the library keeps it
    final = np.array([[oracle.bf16_rne(float(v)) for v in row] for row in r], np.uint16)
    assert np.array_equal(final, out_bits)
    return worst


def free_running(layers, x_bits, out_bits, rec, sample, eps=1e-6, threads=0):
    st = oracle.stack_forward(layers, x_bits[sample], eps=eps, threads=threads)
    diverged = []
    for i, t in enumerate(sample):
        for l in range(len(layers)):
            if set(st["ids"][l, i].tolist()) != set(rec[l]["topk_ids"][t].tolist()):
                diverged.append(int(t))
                break
    keep = [i for i, t in enumerate(sample) if int(t) not in diverged]
    y = synth.bf16_to_f32(out_bits[np.asarray(sample)[keep]]).astype(np.float64)
    ref = synth.bf16_to_f32(st["out"][keep]).astype(np.float64)
    err = row_rel_err(y, ref)
    assert err.max() <= OUT_TOL, err.max()
    return diverged, float(err.max())


def test_stack_3_layers_q4_1_zipf():
    say("case stack3 T=32 q4_1 zipf0.8")
    layers = [synth.make_layer(seed=s, fmt="q4_1", zipf=0.8) for s in range(3)]
    x = synth.make_x(32)
    out, rec = run_stack(layers, x)
    worst = teacher_forced(layers, x, out, rec)
    diverged, err = free_running(layers, x, out, rec, sample=np.arange(32))
    say(f"  teacher-forced max err {worst:.2e}; free-running max err {err:.2e}, diverged {diverged}")


def test_stack_2_layers_nvfp4_and_bf16():
    for fmt in ("nvfp4", "bf16"):
        say(f"case stack2 T=20 {fmt}")
        layers = [synth.make_layer(seed=10 + s, fmt=fmt, zipf=1.1) for s in range(2)]
        x = synth.make_x(20, xseed=5)
        out, rec = run_stack(layers, x)
        teacher_forced(layers, x, out, rec)
        free_running(layers, x, out, rec, sample=np.arange(20))


@pytest.mark.slow
def test_stack47_decode_t32_q4_1_zipf():
    """The 47-layer stack at its full size: ~23.7 GB of q4_1 experts resident."""
    say("case stack47_decode_t32_q4_1_zipf0.8: generating 47 layers")
    layers, x = synth.make_workload("stack47_decode_t32_q4_1_zipf0.8", workers=16,
                                    progress=lambda l: say(f"  layer {l} ready"))
    say("  running the stack on the GPU")
    out, rec = run_stack(layers, x)
    say("  teacher-forced check, every layer")
    worst = teacher_forced(layers, x, out, rec)
    say("  free-running oracle on 8 tokens")
    diverged, err = free_running(layers, x, out, rec, sample=np.array([0, 3, 7, 12, 18, 23, 27, 31]))
    say(f"  teacher-forced max err {worst:.2e}; free-running max err {err:.2e}; diverged {diverged}")
