"""Pins for the oracle's routing, expert FFN, combine, buckets and stack.

What pins what:
  * top-k: brute force over every k-subset (the selected set has the largest
    logit sum), explicit ties, and the (logit desc, id asc) order;
  * weights: the identity renorm(top-k of softmax over E) == softmax(top-k
    logits), and the plain top-k softmax entries when renormalisation is off,
    both against scipy's softmax;
  * router: numpy fp64 matmul of the decoded bf16 operands;
  * layer: a dense evaluation of every expert with numpy (decoded weights,
    fp64 matmuls) mixed by a gate vector that is zero off the top-k; the
    one-expert case reduces to a textbook SwiGLU FFN; k == E gives a dense
    softmax mixture;
  * invariants: relabelling experts, permuting tokens, zero bias, shared-scale
    linearity;
  * buckets: Python's stable sort and bincount;
  * stack: composition of pinned layer calls with numpy RMSNorm;
  * the page's structure: 6 distinct routed experts + 1 shared per token.
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_layer(seed=0, fmt="q4_1", E=8, d=64, f=32, k=2, n_shared=1, zipf=None, renorm=1, shared_scale=1.0):
    return synth.make_layer(seed=seed, fmt=fmt, E=E, d=d, f=f, k=k, n_shared=n_shared, zipf=zipf, renorm=renorm,
                            shared_scale=shared_scale)


def decoded(q, n):
    return oracle.decode_matrix(q, n).astype(np.float64)


def numpy_swiglu(x, Wg, Wu, Wd):
    g = x @ Wg.T
    u = x @ Wu.T
    return (g / (1 + np.exp(-g)) * u) @ Wd.T


def numpy_layer(L, x_bits):
    """Dense reference: every expert evaluated, gates zero off the top-k."""
    x = synth.bf16_to_f32(x_bits).astype(np.float64)
    Wr = synth.bf16_to_f32(L.router_w).astype(np.float64)
    logits = x @ Wr.T + (0 if L.router_b is None else L.router_b.astype(np.float64))
    T = x.shape[0]
    gates = np.zeros((T, L.E))
    for t in range(T):
        order = sorted(range(L.E), key=lambda e: (-logits[t, e], e))[:L.k]
        if L.renorm:
            gates[t, order] = scipy.special.softmax(logits[t, order])
        else:
            gates[t, order] = scipy.special.softmax(logits[t])[order]
    ys = np.stack([numpy_swiglu(x, decoded(L.gate, e), decoded(L.up, e), decoded(L.down, e)) for e in range(L.E)], 1)
    out = np.einsum("te,ted->td", gates, ys)
    if L.n_shared:
        out += L.shared_scale * numpy_swiglu(x, decoded(L.sh_gate, 0), decoded(L.sh_up, 0), decoded(L.sh_down, 0))
    return out, logits


# ---- top-k and weights ------------------------------------------------------------

@pytest.mark.parametrize("E,k", [(8, 2), (12, 3), (16, 4)])
def test_topk_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    for _ in range(50):
        lg = rng.standard_normal(E)
        ids, gap = oracle.topk(lg, k)
        best = max(itertools.combinations(range(E), k), key=lambda s: lg[list(s)].sum())
        assert sorted(ids.tolist()) == sorted(best)
        assert all(lg[ids[j]] >= lg[ids[j + 1]] for j in range(k - 1))
        srt = np.sort(lg)[::-1]
        assert gap == pytest.approx(srt[k - 1] - srt[k], abs=0)


def test_topk_ties_go_to_lower_id():
    lg = np.array([1.0, 3.0, 2.0, 3.0, 2.0, 0.5])
    ids, gap = oracle.topk(lg, 3)
    assert ids.tolist() == [1, 3, 2]
    assert gap == 0.0
    ids, _ = oracle.topk(np.zeros(10), 4)
    assert ids.tolist() == [0, 1, 2, 3]


def test_weights_softmax_identity():
    rng = np.random.default_rng(7)
    for E, k in [(256, 6), (8, 2), (16, 16)]:
        lg = rng.standard_normal(E) * 3
        ids, _ = oracle.topk(lg, k)
        w = oracle.route_weights(lg, ids, renorm=1)
        p = scipy.special.softmax(lg)[ids]
        assert np.allclose(w, p / p.sum(), rtol=0, atol=1e-15)
        assert abs(w.sum() - 1) < 1e-15
        w0 = oracle.route_weights(lg, ids, renorm=0)
        assert np.allclose(w0, scipy.special.softmax(lg)[ids], rtol=0, atol=1e-15)


def test_router_logits_match_numpy():
    L = small_layer(zipf=1.1)
    x = synth.make_x(5, d=L.d, xseed=3)
    r = oracle.route(L, x)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    ref = xf @ synth.bf16_to_f32(L.router_w).astype(np.float64).T + L.router_b.astype(np.float64)
    assert np.allclose(r["logits"], ref, rtol=0, atol=1e-12)


# ---- the layer ----------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["q4_1", "nvfp4", "bf16"])
def test_layer_equals_dense_gated_evaluation(fmt):
    L = small_layer(fmt=fmt, zipf=0.8 if fmt == "nvfp4" else None)
    x = synth.make_x(6, d=L.d, xseed=11)
    r = oracle.layer_forward(L, x)
    ref, logits = numpy_layer(L, x)
    assert np.allclose(r["logits"], logits, rtol=0, atol=1e-12)
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-13)


def test_single_expert_is_textbook_swiglu():
    L = small_layer(E=1, k=1, n_shared=0)
    x = synth.make_x(3, d=L.d, xseed=2)
    r = oracle.layer_forward(L, x)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    ref = numpy_swiglu(xf, decoded(L.gate, 0), decoded(L.up, 0), decoded(L.down, 0))
    assert np.allclose(r["w"], 1.0)
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-14)


def test_k_equals_E_is_dense_softmax_mixture():
    L = small_layer(E=4, k=4, n_shared=0)
    x = synth.make_x(2, d=L.d, xseed=4)
    r = oracle.layer_forward(L, x)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    lg = xf @ synth.bf16_to_f32(L.router_w).astype(np.float64).T
    p = scipy.special.softmax(lg, axis=1)
    ys = [numpy_swiglu(xf, decoded(L.gate, e), decoded(L.up, e), decoded(L.down, e)) for e in range(4)]
    ref = sum(p[:, e:e + 1] * ys[e] for e in range(4))
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-14)


def test_shared_scale_linearity_and_structure():
    x = synth.make_x(4, d=64, xseed=5)
    outs = {s: oracle.layer_forward(small_layer(shared_scale=s), x)["out"] for s in (0.0, 1.0, 2.5)}
    sh = outs[1.0] - outs[0.0]
    assert np.allclose(outs[2.5] - outs[0.0], 2.5 * sh, rtol=1e-12, atol=1e-14)
    L = small_layer()
    xf = synth.bf16_to_f32(x).astype(np.float64)
    ref_sh = numpy_swiglu(xf, decoded(L.sh_gate, 0), decoded(L.sh_up, 0), decoded(L.sh_down, 0))
    assert np.allclose(sh, ref_sh, rtol=1e-12, atol=1e-14)


def test_relabelling_experts_permutes_ids_only():
    L = small_layer(E=8, k=3, zipf=0.5)
    x = synth.make_x(5, d=L.d, xseed=9)
    r = oracle.layer_forward(L, x)
    sigma = np.array([3, 7, 0, 5, 1, 6, 2, 4])  # new id of old expert e is sigma[e]
    inv = np.argsort(sigma)
    P = small_layer(E=8, k=3, zipf=0.5)
    P.router_w = L.router_w[inv].copy()
    P.router_b = L.router_b[inv].copy()
    for name in ("gate", "up", "down"):
        q = getattr(L, name)
        qq = getattr(P, name)
        qq.codes = q.codes[inv].copy()
        qq.scales = q.scales[inv].copy()
    rp = oracle.layer_forward(P, x)
    assert np.array_equal(np.sort(rp["ids"], 1), np.sort(sigma[r["ids"]], 1))
    assert np.allclose(rp["out"], r["out"], rtol=1e-13, atol=1e-15)


def test_token_permutation_and_zero_bias():
    L = small_layer(E=8, k=2)
    x = synth.make_x(7, d=L.d, xseed=12)
    r = oracle.layer_forward(L, x)
    p = np.array([4, 0, 6, 2, 1, 5, 3])
    rp = oracle.layer_forward(L, x[p])
    assert np.array_equal(rp["out"], r["out"][p])
    Lb = small_layer(E=8, k=2)
    Lb.router_b = np.zeros(8, np.float32)
    assert np.array_equal(oracle.layer_forward(Lb, x)["out"], r["out"])


def test_forced_ids_reevaluate_the_given_set():
    L = small_layer(E=8, k=2)
    x = synth.make_x(3, d=L.d, xseed=13)
    forced = np.array([[0, 1], [2, 3], [7, 6]], np.int32)
    r = oracle.layer_forward(L, x, forced_ids=forced)
    assert np.array_equal(r["ids"], forced)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    lg = xf @ synth.bf16_to_f32(L.router_w).astype(np.float64).T
    for t in range(3):
        w = scipy.special.softmax(lg[t, forced[t]])
        ref = sum(w[j] * numpy_swiglu(xf[t:t + 1], decoded(L.gate, e), decoded(L.up, e), decoded(L.down, e))[0]
                  for j, e in enumerate(forced[t]))
        ref += numpy_swiglu(xf[t:t + 1], decoded(L.sh_gate, 0), decoded(L.sh_up, 0), decoded(L.sh_down, 0))[0]
        assert np.allclose(r["out"][t], ref, rtol=1e-12, atol=1e-14)


# ---- buckets ----------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E", [(1, 6, 256), (5, 2, 8), (64, 6, 256), (300, 6, 16), (0, 6, 256)])
def test_buckets_match_stable_sort(T, k, E):
    rng = np.random.default_rng(T + k + E)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32) if T else \
        np.zeros((0, k), np.int32)
    b = oracle.buckets(ids, E)
    flat = ids.reshape(-1)
    S = T * k
    assert np.array_equal(b["counts"], np.bincount(flat, minlength=E))
    assert b["offsets"][0] == 0 and b["offsets"][E] == S
    assert np.array_equal(np.diff(b["offsets"]), b["counts"])
    assert b["perm"].tolist() == sorted(range(S), key=flat.__getitem__)
    assert np.array_equal(b["inv_perm"][b["perm"]], np.arange(S))
    for e in range(E):  # token order ascends inside a bucket
        seg = b["perm"][b["offsets"][e]:b["offsets"][e + 1]] // k
        assert np.all(np.diff(seg) > 0)


# ---- stack ------------------------------------------------------------------------------

def test_rmsnorm_matches_numpy():
    rng = np.random.default_rng(3)
    r = rng.standard_normal(2048) * 3
    got = synth.bf16_to_f32(oracle.rmsnorm_bf16(r, 1e-6)).astype(np.float64)
    ref = r / np.sqrt(np.mean(r * r) + 1e-6)
    # within half a bf16 step: at most 2^-8 relative (8 significant bits)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2 ** -8)
    assert np.abs(got - ref).max() > 0


def test_rmsnorm_eps_inside_the_root_closed_forms():
    """A constant row c has mean square c^2, so RMSNorm gives c / sqrt(c^2 + eps)
    with eps inside the root: 1/sqrt(2) -> bf16 0.70703125 when c^2 = eps
    (eps outside would give c / (c + eps) ~ 0.999 -> bf16 1.0); with eps = 0 it
    is sign(c) exactly; a zero row stays zero."""
    for c in (1e-3, -1e-3):
        got = synth.bf16_to_f32(oracle.rmsnorm_bf16(np.full(2048, c), 1e-6))
        assert np.all(got == np.float32(np.sign(c) * 0.70703125)), got[:4]
    got = synth.bf16_to_f32(oracle.rmsnorm_bf16(np.full(2048, 3e-7), 0.0))
    assert np.all(got == 1.0)
    got = synth.bf16_to_f32(oracle.rmsnorm_bf16(np.zeros(2048), 1e-6))
    assert np.all(got == 0.0)


def test_stack_is_composition_of_layers():
    Ls = [small_layer(seed=s, E=8, k=2, zipf=0.8) for s in range(3)]
    x = synth.make_x(4, d=64, xseed=1)
    st = oracle.stack_forward(Ls, x, eps=1e-6)
    r = synth.bf16_to_f32(x).astype(np.float64)
    for l, L in enumerate(Ls):
        xn = np.stack([oracle.rmsnorm_bf16(row, 1e-6) for row in r])
        assert np.array_equal(xn, st["xin"][l])
        y = oracle.layer_forward(L, xn)
        yb = np.array([[oracle.bf16_rne(v) for v in row] for row in y["out"]], np.uint16)
        assert np.array_equal(yb, st["yout"][l])
        assert np.array_equal(y["ids"], st["ids"][l])
        r = r + synth.bf16_to_f32(yb)
    outb = np.array([[oracle.bf16_rne(v) for v in row] for row in r], np.uint16)
    assert np.array_equal(outb, st["out"])


# ---- the page's structure and closed forms ---------------------------------------------------

def test_page_structure_and_closed_forms():
    pc = {k: v["value"] for k, v in json.load(open(os.path.join(GOLDEN, "page_constants.json"))).items()
          if not k.startswith("_")}
    E, k, n_sh, n_moe = pc["routed_experts_per_moe_layer"], pc["experts_selected_per_token"], \
        pc["shared_experts_always_active"], pc["layers_moe"]
    assert (E, k, n_sh, n_moe) == (256, 6, 1, 47)
    assert pc["layers_total"] - pc["layers_dense"] == n_moe
    d, f = 2048, 512
    per_expert = 3 * d * f
    # per-token active MoE weights and bytes per layer (q4_1 = 5 bits, NVFP4 = 4.5 bits + scales, bf16 = 16)
    L1 = synth.alloc_qmat("q4_1", 1, f, d)
    assert (k + n_sh) * (2 * L1.nbytes() + synth.alloc_qmat("q4_1", 1, d, f).nbytes()) == 13_762_560
    assert (k + n_sh) * 3 * synth.alloc_qmat("bf16", 1, f, d).nbytes() == 44_040_192
    assert (k + n_sh) * 3 * synth.alloc_qmat("nvfp4", 1, f, d).nbytes() == 12_386_304 + 84
    # totals stay inside the page's parameter counts
    moe_total = n_moe * ((E + n_sh) * per_expert + E * d)
    moe_active = n_moe * ((k + n_sh) * per_expert + E * d)
    assert moe_total <= pc["params_total"] and moe_total / pc["params_total"] > 0.9
    assert moe_active <= pc["params_active_body"]
    # storage bits per weight order the formats as the page's file sizes do
    bits = {fmt: 8 * synth.alloc_qmat(fmt, 1, f, d).nbytes() / (f * d) for fmt in ("q4_1", "nvfp4", "bf16")}
    assert bits["q4_1"] == 5.0 and abs(bits["nvfp4"] - 4.5) < 1e-4 and bits["bf16"] == 16
    assert pc["file_bytes_q4_1_gguf"] > pc["file_bytes_nvfp4_gguf"]
    assert abs(pc["file_bytes_bf16"] / pc["params_total"] - 2.0) < 0.01


def test_each_token_uses_six_distinct_routed_experts_and_the_shared_one():
    L = small_layer(E=16, k=6)
    x = synth.make_x(9, d=L.d, xseed=21)
    r = oracle.layer_forward(L, x)
    for t in range(9):
        assert len(set(r["ids"][t].tolist())) == 6
        assert np.all((0 <= r["ids"][t]) & (r["ids"][t] < 16))
    # the shared expert acts on every token: removing it changes every row
    r0 = oracle.layer_forward(small_layer(E=16, k=6, n_shared=0), x)
    assert np.all(np.abs(r["out"] - r0["out"]).max(1) > 0)


@pytest.mark.slow
def test_full_size_uniform_routing_touches_expected_expert_count():
    """At d=2048 the unbiased router gives near-uniform load: over the 64-token
    decode batch the number of distinct experts touched sits near the
    uniform-routing value 256 * (1 - (250/256)^64) = 199.9 (sd ~ 6.6)."""
    L = synth.make_layer(seed=0, fmt="q4_1")
    x = synth.make_x(64)
    r = oracle.route(L, x)
    U = len(np.unique(r["ids"]))
    assert abs(U - 256 * (1 - (250 / 256) ** 64)) < 4 * 6.6
