"""GPU-vs-oracle comparison rules shared by the GPU tests (not a test module).

Rules (eps = 1e-4 on the oracle's fp64 logits, bias included; for a token row
whose RMS exceeds 1 the logit, gap and weight tolerances grow with that RMS,
since fp32 accumulation errors are relative to the row's size):
  * expert ids: the GPU set S is accepted iff min_{e in S} L_e >= max_{e not in S} L_e - eps.
    Where the oracle's k-th to (k+1)-th gap exceeds eps this forces S to equal the
    oracle's set exactly; inside a near-tie either choice is valid.  The order in S
    is checked where adjacent oracle logits differ by more than eps.
  * routing weights: |w_gpu - w_oracle(S_gpu)| <= 1e-5.
  * logits: |L_gpu - L_oracle| <= 1e-4 (fp32 accumulation of 2048 bf16 products).
  * buckets: counts, offsets, perm and inv_perm equal the oracle's bucketing of
    the GPU ids bit for bit.
  * outputs: per token row, max_j |y_j - r_j| / max_j |r_j| <= 1e-2, with r the
    oracle's layer on the same token routed to the GPU's set (the weights of
    that set come from the oracle's own logits).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import quantized_expert_ffn_wave_amd as moe
import synth

EPS = 1e-4
W_TOL = 1e-5
LOGIT_TOL = 1e-4
OUT_TOL = 1e-2


def say(msg: str) -> None:
    print(msg, flush=True)


def x_to_dev(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def row_rel_err(y: np.ndarray, r: np.ndarray) -> np.ndarray:
    den = np.maximum(np.abs(r).max(1), 1e-30)
    return np.abs(y - r).max(1) / den


def gpu_forward(dl: moe.DeviceLayer, x_bits: np.ndarray, E: int, k: int, persistent: bool = False):
    T = x_bits.shape[0]
    route, bufs = moe.route_buffers(T, k, E)
    x = x_to_dev(x_bits)
    y = moe.layer_forward(dl, x, route=route, persistent=persistent)
    torch.cuda.synchronize()
    out = {n: t.cpu().numpy() for n, t in bufs.items() if n not in ("x_in", "y_out")}
    out["perm"] = out["perm"][:T * k]
    out["inv_perm"] = out["inv_perm"][:T * k]
    out["y_bits"] = bits_of(y)
    out["x_in_bits"] = bits_of(bufs["x_in"])
    out["y_out_bits"] = bits_of(bufs["y_out"])
    return out


def row_scale(x_bits: np.ndarray) -> np.ndarray:
    """max(1, RMS) of each bf16 token row: the factor the routing tolerances take."""
    x = synth.bf16_to_f32(x_bits).astype(np.float64)
    return np.maximum(1.0, np.sqrt(np.mean(x * x, axis=1)))


def check_routing(g: dict, o: dict, E: int, k: int, scale: np.ndarray | None = None) -> dict:
    """Apply the id/weight/logit/bucket rules; returns counts of near-tie tokens.
    scale: per token, the factor of the tolerances (row_scale; default 1)."""
    T = g["topk_ids"].shape[0]
    L = o["logits"]
    sc = np.ones(T) if scale is None else np.asarray(scale, np.float64)
    dl = np.abs(g["logits"] - L).max(axis=1) if T else np.zeros(0)
    assert np.all(dl <= LOGIT_TOL * sc), (dl / sc).max()
    ties = 0
    for t in range(T):
        eps = EPS * sc[t]
        S = g["topk_ids"][t]
        assert len(set(S.tolist())) == k and S.min() >= 0 and S.max() < E, (t, S)
        mask = np.zeros(E, bool)
        mask[S] = True
        if k < E:
            assert L[t, mask].min() >= L[t, ~mask].max() - eps, (t, S, o["ids"][t])
        if o["gaps"][t] > eps:
            assert set(S.tolist()) == set(o["ids"][t].tolist()), (t, S, o["ids"][t])
        else:
            ties += 1
        for j in range(k - 1):
            if L[t, S[j]] - L[t, S[j + 1]] < -eps:
                raise AssertionError(f"token {t}: order {S} not logit-descending")
        ref_w = oracle.route_weights(L[t], S, renorm=o.get("renorm", 1))
        assert np.abs(g["topk_w"][t] - ref_w).max() <= W_TOL * sc[t], (t, g["topk_w"][t], ref_w)
    b = oracle.buckets(g["topk_ids"], E)
    assert np.array_equal(g["counts"], b["counts"])
    assert np.array_equal(g["offsets"], b["offsets"])
    assert np.array_equal(g["perm"], b["perm"])
    assert np.array_equal(g["inv_perm"], b["inv_perm"])
    return dict(ties=ties)


def check_layer(host, x_bits: np.ndarray, dl: moe.DeviceLayer | None = None, sample=None, tol: float = OUT_TOL,
                threads: int = 0, persistent: bool = False) -> dict:
    """Run the GPU layer (persistent: the persistent decode path) and compare it
    with the oracle under the rules above."""
    if dl is None:
        dl = moe.DeviceLayer(host, max_tokens=max(x_bits.shape[0], 1))
    g = gpu_forward(dl, x_bits, host.E, host.k, persistent=persistent)
    assert np.array_equal(g["x_in_bits"], x_bits)
    assert np.array_equal(g["y_out_bits"], g["y_bits"])
    o = oracle.route(host, x_bits, threads=threads)
    o["renorm"] = host.renorm
    info = check_routing(g, o, host.E, host.k, scale=row_scale(x_bits))
    toks = np.arange(x_bits.shape[0]) if sample is None else np.asarray(sample)
    ref = oracle.layer_forward(host, x_bits[toks], forced_ids=g["topk_ids"][toks], threads=threads)
    y = synth.bf16_to_f32(g["y_bits"][toks]).astype(np.float64)
    err = row_rel_err(y, ref["out"])
    assert np.all(np.isfinite(y))
    assert err.max() <= tol, (err.max(), int(err.argmax()))
    info.update(max_err=float(err.max()), mean_err=float(err.mean()), counts=g["counts"], gpu=g)
    return info
