#!/usr/bin/env python3
"""Throughput of the MoE-layer forward on one MI355X.

A step is one pass of the whole layer (router, top-k, buckets, gate/up +
SwiGLU, down, combine; the shared expert in the same work lists) over
one batch of synthetic tokens.  Steps are timed as HIP-graph replays of the
library's forward (one captured graph per layer instance; the forward is
capturable because it never synchronises the host), which is how a decode
loop launches it; `--no-graph` times plain launches instead.  Per-kernel
durations for the roofline come from a second timed region of plain
launches with HIP events recorded between the kernels on the library's
stream (event records inside a captured graph do not time kernels).  The default
workload is the 64-token decode layer with q4_1 experts (256 routed + 1 shared,
width 512, d_model 2048, top-6, near-uniform routing).  Steps rotate over
`--layers` independently drawn layer instances (3.9 GB of packed weights for 8)
so that every step reads its expert weights from HBM, not from the 256 MB
last-level cache.

Prints one JSON line: tokens/s (the metric), the achieved HBM bandwidth on the
expert-weight bytes the step touches, a roofline entry for the dominant kernel
(gate/up + SwiGLU) timed with HIP events on the library's stream, and the CPU
oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("ffn.hip", "common.hpp"):
        with open(os.path.join(ROOT, "quantized_expert_ffn_wave_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per gate/up launch from the committed counter summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(PROFILE_DIR, f"ffn_up_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_t64_q4_1")
    ap.add_argument("--layers", type=int, default=8, help="layer instances the steps rotate over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time plain launches instead of HIP-graph replays")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import quantized_expert_ffn_wave_amd as moe
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    cfg = synth.CONFIGS[args.workload]
    if cfg["layers"] != 1:
        print("bench.py times single-layer workloads", file=sys.stderr)
        return 2
    T, fmt = cfg["T"], cfg["fmt"]
    NL = max(1, args.layers)

    log(f"generating {NL} layer instances of {args.workload}")
    t0 = time.time()
    hosts = []
    for s in range(NL):
        hosts.append(synth.make_layer(seed=s, fmt=fmt, zipf=cfg["zipf"]))
        log(f"  layer {s} ready ({time.time() - t0:.1f} s)")
    x_bits = synth.make_x(T)
    dls = [moe.DeviceLayer(h, max_tokens=T) for h in hosts]
    x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    y = torch.empty_like(x)
    ws = moe.alloc_workspace(dls[0].workspace_size(T))
    stream = moe.current_stream()
    E, K = hosts[0].E, hosts[0].k

    # routing of each instance (untimed): touched experts -> algorithmic bytes
    exp_b = hosts[0].expert_bytes()
    gu_b = hosts[0].gate.nbytes() + hosts[0].up.nbytes()
    dn_b = hosts[0].down.nbytes()
    S = T * K
    touched, step_w_bytes, up_bytes = [], [], []
    for dl in dls:
        route, bufs = moe.route_buffers(T, K, E)
        moe.layer_forward(dl, x, y, route=route, workspace=ws)
        torch.cuda.synchronize()
        U = int((bufs["counts"].cpu().numpy() > 0).sum())
        touched.append(U)
        step_w_bytes.append((U + 1) * exp_b)
        # gate/up launch: the gate and up matrices of the touched experts and
        # the shared one, the tokens once, the SwiGLU rows of the S + T slots
        up_bytes.append((U + 1) * gu_b + T * 2048 * 2 + (S + T) * 512 * 2)
    router_b = E * 2048 * 2

    def step(i, events=None, on=None):
        dl = dls[i % NL]
        if events is None:
            moe.moe_layer_forward(dl.handle, x.data_ptr(), T, y.data_ptr(), None, ws.data_ptr(), ws.numel(),
                                  stream if on is None else on)
        else:
            moe.moe_layer_forward_staged(dl.handle, x.data_ptr(), T, y.data_ptr(), None, ws.data_ptr(), ws.numel(),
                                         stream, events)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # per-step stage events, created and recorded once so the handles exist
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(moe.N_STAGE_EVENTS)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    handles = [[e.cuda_event for e in row] for row in evs]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i, handles[i])
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms = total_ms / args.steps

    graph_ms = None
    if not args.no_graph:
        graphs = []
        for i in range(NL):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i, on=moe.current_stream())
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % NL].replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for i in range(args.steps):
            graphs[(args.warmup + i) % NL].replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        log(f"graph replay: {graph_ms * 1e3:.1f} us per step")

    stage_ms = np.array([[row[j].elapsed_time(row[j + 1]) for j in range(moe.N_STAGE_EVENTS - 1)] for row in evs])
    idx = [(args.warmup + i) % NL for i in range(args.steps)]
    up_ms = stage_ms[:, moe.STAGES.index("gate_up")]
    up_achieved = sum(up_bytes[j] for j in idx) / (up_ms.sum() * 1e-3) / 1e9
    w_bytes = float(np.mean([step_w_bytes[j] for j in idx]))
    step_ms = graph_ms if graph_ms is not None else ms
    gbps = w_bytes / (step_ms * 1e-3) / 1e9
    traffic = read_traffic(args.workload)
    stage_means = {n: round(float(v), 4) for n, v in zip(moe.STAGES, stage_ms.mean(0))}
    log(f"stage means (ms): {stage_means}")

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {n} bytes")
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # bounded sample: whole steps (the full batch through one layer
        # instance, cycling over the instances) until about 10 s have passed
        th = oracle.max_threads()
        log(f"cpu baseline: oracle on {th} threads, whole {T}-token steps for about 10 s")
        n_cpu, c0 = 0, time.time()
        while n_cpu < 1 or (time.time() - c0 < 10.0 and n_cpu < 64):
            oracle.layer_forward(hosts[n_cpu % NL], x_bits, threads=th)
            n_cpu += 1
        dt = time.time() - c0
        cpu = {"value": round(n_cpu * T / dt, 3), "unit": "tokens/s", "cores": th, "kind": "oracle",
               "sample": f"{n_cpu} steps of the same workload (the full {T}-token batch through one layer "
                         f"instance each; fp64 routing and 7 experts per token), {dt:.1f} s wall"}

    out = {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s (% of peak), decode batch 1\u2013256, 1 GPU",
        "value": round(T / (step_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{fmt} weights, f16 operands, f32 accumulate",
        "data": "synthetic",
        "hbm_gbps_expert_weights": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "config": {"workload": f"moe_layer_{args.workload}", "tokens": T, "d_model": 2048, "routed_experts": E,
                   "top_k": K, "shared_experts": 1, "d_expert": 512, "weights": fmt, "router_bias_zipf": cfg["zipf"],
                   "layer_instances": NL, "touched_experts_mean": round(float(np.mean(touched)), 1),
                   "expert_weight_bytes_per_step": int(w_bytes), "router_bytes_per_step": router_b,
                   "launch": "hip_graph_replay" if graph_ms is not None else "plain",
                   "plain_launch_ms_per_step": round(ms, 5), "stage_ms": stage_means},
        "roofline": {"bound": "hbm", "kernel": "ffn_up_kernel (gate/up + SwiGLU)",
                     "achieved": round(up_achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(up_achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    for d in dls:
        d.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
