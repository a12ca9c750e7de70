#!/usr/bin/env python3
"""Throughput of the MoE-layer forward on one MI355X.

A step is one pass of the whole layer (router, top-k, buckets, gate/up +
SwiGLU, down, combine; the shared expert in the same work lists) over
one batch of synthetic tokens.  Steps are timed as HIP-graph replays of the
library's forward (one captured graph holds a forward of each layer instance
in turn, as a decode loop captures its whole step; the forward is capturable
because it never synchronises the host); `--no-graph` times plain launches
instead.  Per-kernel
durations for the roofline come from a second timed region of plain
launches with HIP events recorded between the kernels on the library's
stream (event records inside a captured graph do not time kernels).  The default
workload is the 64-token decode layer with q4_1 experts (256 routed + 1 shared,
width 512, d_model 2048, top-6, near-uniform routing).  Steps rotate over
`--layers` independently drawn layer instances (3.9 GB of packed weights for 8)
and, for small batches, over several token sets per instance, so that one
cycle of steps reads at least 1 GiB of expert weights and every step reads its
weights from HBM, not from the 256 MB last-level cache.

The 47-layer workload (`--workload stack47_decode_t32_q4_1_zipf0.8`) times the
pre-norm residual stack instead: a step is 32 tokens through all 47 layers
(23.75 GB of q4_1 weights resident), replayed as one captured graph from the
same input each time; its roofline entry times the gate/up kernel of every
layer on the layer inputs the stack produced.

The output-head workloads (`--workload head_v151552_t4_q4_1` and the others
of synth.HEAD_CONFIGS) time the 4-bit output head instead: a step is the
logits of T tokens against a synthetic 151552 x 2048 head, rotating over
`--layers` drawn heads; its roofline entry is the head kernel itself.  The
decode-attention workloads (`--workload attn_full_b32_ctx8192`,
`attn_swa_b32_ctx8192`) time one attention layer's step for 32 sequences with
8192 cached positions (full attention, or the 513-token window with rotary
embedding).

Also measured, outside the timed steps: the attainable HBM read rate (a plain
streaming read of 4 GiB through the library's moe_stream_read, best of a few
launch shapes), the spread of single graph replays (p10/p50/p90), and for the
64-token q4_1 workload a token-count sweep 1, 2, 4, ..., 256 with the same
generator (`--no-sweep` skips it).

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
MFMA_PEAK_TFLOPS = 2500.0  # dense f16 / bf16 matrix-core peak
PROFILE_DIR = os.path.join(ROOT, "profiles")
STREAM_BYTES = 4 << 30
SWEEP_T = [1, 2, 4, 8, 16, 32, 64, 128, 256]
# One cycle of timed forwards reads at least this many bytes of expert weights
# (four times the chip's 256 MB last-level cache), so that no step finds its
# weights still cached from the previous cycle; small batches get more token
# sets per layer instance to reach it.
CYCLE_MIN_BYTES = 1 << 30
MAX_X_SETS = 16
STACK_EPS = 1e-6


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str = "ffn_up") -> str:
    """Hash of the sources of the kernel a traffic summary was taken on."""
    h = hashlib.sha256()
    files = (("attention.hip", "attention.hpp", "common.hpp") if kernel == "attn" else
             ("layer.hip", "routing.hip", "ffn.hip", "decode.hip", "common.hpp"))
    for f in files:
        with open(os.path.join(ROOT, "quantized_expert_ffn_wave_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_counter_summary(workload: str, kernel: str = "ffn_up") -> dict:
    """Fields of the committed counter summary of the roofline kernel (gate/up,
    or the head), if it was taken on the current kernel source (else {})."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return {}
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv if kv.get("kernel_source_sha") == kernel_source_hash(kernel) else {}


def read_traffic(workload: str, kernel: str = "ffn_up"):
    """HBM bytes per launch of the roofline kernel from the counter summary (or None)."""
    try:
        return float(read_counter_summary(workload, kernel)["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_mfma_busy(workload: str, kernel: str = "ffn_up"):
    """Matrix-core busy fraction of the roofline kernel from the counter summary
    (SQ_VALU_MFMA_BUSY_CYCLES over the SIMD cycles of GRBM_GUI_ACTIVE), or None."""
    try:
        return float(read_counter_summary(workload, kernel)["mfma_busy"])
    except (KeyError, ValueError):
        return None


def operand_dtype(fmt: str) -> str:
    """What the expert products compute in, for a weight format."""
    if fmt == "bf16":
        return "bf16 weights, bf16 operands, f32 accumulate"
    return f"{fmt} weights, f16 operands (per-token power-of-two scaled), f32 accumulate"


def pct(a, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(a), q)), 5)


def stream_reference(moe, torch):
    """Attainable HBM read rate: best of a few launch shapes of a plain 4 GiB read."""
    src = torch.empty(STREAM_BYTES, dtype=torch.uint8, device="cuda")
    src.fill_(7)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    stream = moe.current_stream()
    best = None
    for wg_per_cu in (1, 2, 4, 8):
        grid = n_cu * wg_per_cu
        moe.moe_stream_read(src.data_ptr(), STREAM_BYTES, sink.data_ptr(), grid, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            moe.moe_stream_read(src.data_ptr(), STREAM_BYTES, sink.data_ptr(), grid, stream)
        e1.record()
        torch.cuda.synchronize()
        gbps = STREAM_BYTES * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        log(f"stream read 4 GiB, {grid} workgroups: {gbps:.0f} GB/s")
        if best is None or gbps > best[0]:
            best = (gbps, grid)
    del src, sink
    torch.cuda.empty_cache()
    return {"gbps": round(best[0], 1), "bytes": STREAM_BYTES, "workgroups": best[1],
            "kernel": "moe_stream_read (16 B nontemporal loads, 8 in flight per thread)"}


def replay_spread(torch, replay, n):
    """Per-replay durations (ms) with an event pair around each replay."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        evs[i][0].record()
        replay(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def copy_calibration(torch):
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


def bench_layer(args, moe, synth, torch, np):
    cfg = synth.CONFIGS[args.workload]
    T, fmt = cfg["T"], cfg["fmt"]
    NL = max(1, args.layers)
    do_sweep = (not args.no_sweep) and args.workload == "decode_t64_q4_1"
    max_tokens = max(T, SWEEP_T[-1]) if do_sweep else T

    log(f"generating {NL} layer instances of {args.workload}")
    t0 = time.time()
    hosts = []
    for s in range(NL):
        hosts.append(synth.make_layer(seed=s, fmt=fmt, zipf=cfg["zipf"]))
        log(f"  layer {s} ready ({time.time() - t0:.1f} s)")
    x_bits = synth.make_x(T)
    dls = [moe.DeviceLayer(h, max_tokens=max_tokens) for h in hosts]
    x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    y = torch.empty_like(x)
    ws = moe.alloc_workspace(dls[0].workspace_size(T))
    stream = moe.current_stream()
    E, K = hosts[0].E, hosts[0].k

    exp_b = hosts[0].expert_bytes()
    h_elem = 2 if fmt == "bf16" else 4
    gu_b = hosts[0].gate.nbytes() + hosts[0].up.nbytes()

    def touched_bytes(dl, xt, wst):
        """Routing of one instance (untimed): touched experts -> algorithmic bytes."""
        n = xt.shape[0]
        route, bufs = moe.route_buffers(n, K, E)
        moe.layer_forward(dl, xt, torch.empty_like(xt), route=route, workspace=wst)
        torch.cuda.synchronize()
        U = int((bufs["counts"].cpu().numpy() > 0).sum())
        # gate/up launch: the gate and up matrices of the touched experts and
        # the shared one, the tokens once, the SwiGLU rows of the S + T slots
        # (fp32 for the 4-bit formats, bf16 for bf16 weights)
        return U, (U + 1) * exp_b, (U + 1) * gu_b + n * 2048 * 2 + (n * K + n) * 512 * h_elem

    # the timed forwards cycle over (layer instance, token set) pairs; token
    # set 0 is x, the others are drawn with further seeds, as many as a cycle
    # needs to read CYCLE_MIN_BYTES of expert weights
    first_w = [touched_bytes(dl, x, ws)[1] for dl in dls]
    R = min(MAX_X_SETS, max(1, -(-CYCLE_MIN_BYTES // int(sum(first_w)))))
    xs = [x] + [torch.from_numpy(synth.make_x(T, xseed=r).view(np.int16)).cuda().view(torch.bfloat16)
                for r in range(1, R)]
    pairs = [(l, r) for r in range(R) for l in range(NL)]
    P = len(pairs)
    touched, step_w_bytes, up_bytes = [], [], []
    for l, r in pairs:
        U, wb, ub = touched_bytes(dls[l], xs[r], ws)
        touched.append(U)
        step_w_bytes.append(wb)
        up_bytes.append(ub)
    log(f"{R} token set(s) per instance: {P} forwards, {sum(step_w_bytes) / 1e9:.2f} GB of expert weights per cycle")
    router_b = E * 2048 * 2

    def step(i, events=None, on=None):
        l, r = pairs[i % P]
        dl, xr = dls[l], xs[r]
        if events is None:
            fwd = moe.moe_layer_forward_persistent if args.persistent else moe.moe_layer_forward
            fwd(dl.handle, xr.data_ptr(), T, y.data_ptr(), None, ws.data_ptr(), ws.numel(), stream if on is None else on)
        else:
            moe.moe_layer_forward_staged(dl.handle, xr.data_ptr(), T, y.data_ptr(), None, ws.data_ptr(), ws.numel(),
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
    ms = start.elapsed_time(stop) / args.steps

    graph_ms, spread = None, None
    if not args.no_graph:
        # One graph holds a forward of every (instance, token set) pair in
        # turn, as a decode loop captures its whole step rather than one graph
        # per layer (a graph launch costs about 5 us of idle GPU between
        # graphs); a second graph holds the first K % P pairs, so that exactly
        # K steps are timed.
        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    step(i, on=moe.current_stream())
            return g
        n_full, n_rest = divmod(args.steps, P)
        g_all = capture(P)
        g_rest = capture(n_rest) if n_rest else None
        for _ in range(max(1, args.warmup // P)):
            g_all.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(n_full):
            g_all.replay()
        if g_rest is not None:
            g_rest.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        log(f"graph replay: {graph_ms * 1e3:.1f} us per step")
        sp = [v / P for v in replay_spread(torch, lambda i: g_all.replay(), max(n_full, 10))]
        spread = {"p10": pct(sp, 10), "p50": pct(sp, 50), "p90": pct(sp, 90), "steps_per_replay": P}
        del g_all, g_rest

    stage_ms = np.array([[row[j].elapsed_time(row[j + 1]) for j in range(moe.N_STAGE_EVENTS - 1)] for row in evs])
    idx = [(args.warmup + i) % P for i in range(args.steps)]
    up_ms = stage_ms[:, moe.STAGES.index("gate_up")]
    up_flops = 2.0 * (T * K + T) * 2 * 512 * 2048  # gate and up products of every slot
    up_achieved = sum(up_bytes[j] for j in idx) / (up_ms.sum() * 1e-3) / 1e9
    step_ms = graph_ms if graph_ms is not None else ms
    # the timed steps: pairs 0, 1, ... in the graph, warmup, warmup + 1, ... in plain launches
    first = 0 if graph_ms is not None else args.warmup
    w_bytes = float(np.mean([step_w_bytes[(first + i) % P] for i in range(args.steps)]))
    gbps = w_bytes / (step_ms * 1e-3) / 1e9
    traffic = read_traffic(args.workload)
    stage_means = {n: round(float(v), 4) for n, v in zip(moe.STAGES, stage_ms.mean(0))}
    log(f"stage means (ms): {stage_means}")

    sweep = None
    if do_sweep:
        sweep = []
        x_all = torch.from_numpy(synth.make_x(SWEEP_T[-1]).view(np.int16)).cuda().view(torch.bfloat16)
        ws_all = moe.alloc_workspace(max(dls[0].workspace_size(t) for t in SWEEP_T))
        for t in SWEEP_T:
            # token sets: disjoint row windows of x_all, as many as a cycle over
            # the instances needs to read CYCLE_MIN_BYTES (see the timed steps)
            yt = torch.empty((t, 2048), dtype=torch.bfloat16, device="cuda")
            tb0 = [touched_bytes(dl, x_all[:t].contiguous(), ws_all)[1] for dl in dls]
            Rt = min(MAX_X_SETS, SWEEP_T[-1] // t, max(1, -(-CYCLE_MIN_BYTES // int(sum(tb0)))))
            xts = [x_all[r * t:(r + 1) * t].contiguous() for r in range(Rt)]
            tb = [touched_bytes(dl, xr, ws_all) for xr in xts for dl in dls]
            g = torch.cuda.CUDAGraph()  # every (token set, instance) pair in turn, as for the timed steps
            with torch.cuda.graph(g):
                fwd = (moe.moe_layer_forward_persistent if args.persistent and t <= moe.PERSISTENT_MAX_T
                       else moe.moe_layer_forward)
                for xr in xts:
                    for dl in dls:
                        fwd(dl.handle, xr.data_ptr(), t, yt.data_ptr(), None, ws_all.data_ptr(), ws_all.numel(),
                            moe.current_stream())
            n_fwd = Rt * NL
            for _ in range(max(1, args.warmup // n_fwd)):
                g.replay()
            torch.cuda.synchronize()
            reps = max(2, args.steps // (2 * n_fwd))
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            for _ in range(reps):
                g.replay()
            a1.record()
            torch.cuda.synchronize()
            t_ms = a0.elapsed_time(a1) / (reps * n_fwd)
            wb = float(np.mean([b for _, b, _ in tb]))
            sweep.append({"tokens": t, "us_per_step": round(t_ms * 1e3, 2), "tokens_per_s": round(t / (t_ms * 1e-3), 1),
                          "touched_experts_mean": round(float(np.mean([u for u, _, _ in tb])), 1),
                          "hbm_gbps_expert_weights": round(wb / (t_ms * 1e-3) / 1e9, 1),
                          "token_sets": Rt, "weight_bytes_per_cycle": int(sum(b for _, b, _ in tb))})
            log(f"sweep T={t}: {t_ms * 1e3:.1f} us, {sweep[-1]['hbm_gbps_expert_weights']} GB/s")
            del g
        del x_all, ws_all

    if args.copy_calibration:
        copy_calibration(torch)

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

    for d in dls:
        d.close()
    del dls, ws, x, y
    torch.cuda.empty_cache()
    stream_ref = None if args.no_stream_reference else stream_reference(moe, torch)

    out = {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s (% of peak), decode batch 1–256, 1 GPU",
        "value": round(T / (step_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": operand_dtype(fmt),
        "data": "synthetic",
        "hbm_gbps_expert_weights": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "hbm_frac_of_stream_read": round(gbps / stream_ref["gbps"], 4) if stream_ref else None,
        "stream_read": stream_ref,
        "config": {"workload": f"moe_layer_{args.workload}", "tokens": T, "d_model": 2048, "routed_experts": E,
                   "top_k": K, "shared_experts": 1, "d_expert": 512, "weights": fmt, "router_bias_zipf": cfg["zipf"],
                   "layer_instances": NL, "token_sets": R, "touched_experts_mean": round(float(np.mean(touched)), 1),
                   "expert_weight_bytes_per_step": int(w_bytes), "router_bytes_per_step": router_b,
                   "launch": ("hip_graph_replay" if graph_ms is not None else "plain") + (", persistent" if args.persistent else ""),
                   "plain_launch_ms_per_step": round(ms, 5), "graph_replay_ms": spread, "stage_ms": stage_means},
        "roofline": {"bound": "hbm", "kernel": "ffn_up_kernel (gate/up + SwiGLU)",
                     "achieved": round(up_achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(up_achieved / HBM_PEAK_GBPS, 4),
                     "frac_of_stream_read": round(up_achieved / stream_ref["gbps"], 4) if stream_ref else None,
                     "traffic": traffic},
        # the same kernel against the matrix cores: algorithmic products (both
        # matrices over every slot, routed and shared) per event-timed launch,
        # and the busy fraction the committed counter summary measured
        "mfma": {"kernel": "ffn_up_kernel", "operands": "bf16" if fmt == "bf16" else "f16",
                 "achieved_tflops": round(up_flops * len(idx) / (up_ms.sum() * 1e-3) / 1e12, 2),
                 "peak_tflops": MFMA_PEAK_TFLOPS,
                 "frac": round(up_flops * len(idx) / (up_ms.sum() * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
                 "mfma_util": read_mfma_busy(args.workload)},
        "cpu_baseline": cpu,
    }
    if sweep is not None:
        out["token_sweep"] = sweep
    return out


def bench_stack(args, moe, synth, torch, np):
    cfg = synth.CONFIGS[args.workload]
    T, fmt, NLAY = cfg["T"], cfg["fmt"], cfg["layers"]
    log(f"generating the {NLAY} layers of {args.workload}")
    t0 = time.time()
    hosts, x_bits = synth.make_workload(args.workload, workers=16,
                                        progress=lambda l: log(f"  layer {l} ready ({time.time() - t0:.1f} s)"))
    dls = []
    for l, h in enumerate(hosts):
        dls.append(moe.DeviceLayer(h, max_tokens=T))
        if l % 8 == 7:
            log(f"  {l + 1} layers on the device")
    handles = [d.handle for d in dls]
    E, K = hosts[0].E, hosts[0].k
    exp_b = hosts[0].expert_bytes()
    h_elem = 2 if fmt == "bf16" else 4
    gu_b = hosts[0].gate.nbytes() + hosts[0].up.nbytes()
    x0 = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    x = x0.clone()
    ws = moe.alloc_workspace(moe.moe_stack_workspace_size(handles, T))
    stream = moe.current_stream()

    # one untimed pass recording every layer's routing and normalised input
    rb = [moe.route_buffers(T, K, E) for _ in range(NLAY)]
    moe.moe_stack_forward(handles, x.data_ptr(), T, STACK_EPS, [r for r, _ in rb], ws.data_ptr(), ws.numel(), stream)
    torch.cuda.synchronize()
    touched = [int((b["counts"].cpu().numpy() > 0).sum()) for _, b in rb]
    w_bytes = float(sum((u + 1) * exp_b for u in touched))
    up_bytes = [(u + 1) * gu_b + T * 2048 * 2 + (T * K + T) * 512 * (2 if fmt == "bf16" else 4) for u in touched]
    xin = [b["x_in"] for _, b in rb]
    log(f"touched experts per layer: mean {np.mean(touched):.1f}; expert bytes per step {w_bytes / 1e6:.1f} MB")

    def run(on):
        moe.moe_stack_forward(handles, x.data_ptr(), T, STACK_EPS, None, ws.data_ptr(), ws.numel(), on,
                              persistent=args.persistent)

    for _ in range(args.warmup):
        x.copy_(x0)
        run(stream)
    torch.cuda.synchronize()

    def plain(i):
        run(stream)

    # restore outside the event pair so that only the stack pass is timed
    def timed(f, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            x.copy_(x0)
            evs[i][0].record()
            f(i)
            evs[i][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    log(f"timing {args.steps} plain-launch stack steps")
    plain_ms = timed(plain, args.steps)
    ms = float(np.mean(plain_ms))

    graph_ms, spread = None, None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        x.copy_(x0)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            run(moe.current_stream())
        for _ in range(args.warmup):
            x.copy_(x0)
            g.replay()
        torch.cuda.synchronize()
        log(f"timing {args.steps} graph replays of the stack")
        gm = timed(lambda i: g.replay(), args.steps)
        graph_ms = float(np.mean(gm))
        spread = {"p10": pct(gm, 10), "p50": pct(gm, 50), "p90": pct(gm, 90)}
        log(f"graph replay: {graph_ms * 1e3:.1f} us per 47-layer step")
        # the replay reproduces the recorded pass (same input, same routing)
        x_chk = x.clone()
        x.copy_(x0)
        run(stream)
        torch.cuda.synchronize()
        if not torch.equal(x_chk, x):
            raise RuntimeError("graph replay of the stack differs from a plain pass")
        del g

    # roofline: the gate/up stage of every layer on the inputs the stack produced,
    # one layer after another so that each reads its weights from HBM
    y = torch.empty_like(x)
    wsl = moe.alloc_workspace(dls[0].workspace_size(T))
    n_rep = max(1, args.steps // 10)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(moe.N_STAGE_EVENTS)] for _ in range(NLAY * n_rep)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for r in range(n_rep):
        for l in range(NLAY):
            row = [e.cuda_event for e in evs[r * NLAY + l]]
            moe.moe_layer_forward_staged(handles[l], xin[l].data_ptr(), T, y.data_ptr(), None, wsl.data_ptr(),
                                         wsl.numel(), stream, row)
    torch.cuda.synchronize()
    stage_ms = np.array([[row[j].elapsed_time(row[j + 1]) for j in range(moe.N_STAGE_EVENTS - 1)] for row in evs])
    up_ms = stage_ms[:, moe.STAGES.index("gate_up")]
    up_flops = 2.0 * (T * K + T) * 2 * 512 * 2048  # gate and up products of every slot
    up_achieved = n_rep * sum(up_bytes) / (up_ms.sum() * 1e-3) / 1e9
    stage_means = {n: round(float(v), 4) for n, v in zip(moe.STAGES, stage_ms.mean(0))}
    log(f"per-layer stage means (ms): {stage_means}")

    step_ms = graph_ms if graph_ms is not None else ms
    gbps = w_bytes / (step_ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        th = oracle.max_threads()
        n_tok = 8
        log(f"cpu baseline: oracle stack on {th} threads, {n_tok} tokens through all {NLAY} layers, about 10 s")
        n_cpu, c0 = 0, time.time()
        while n_cpu < 1 or (time.time() - c0 < 10.0 and n_cpu < 16):
            sl = slice((n_cpu * n_tok) % T, (n_cpu * n_tok) % T + n_tok)
            oracle.stack_forward(hosts, x_bits[sl], eps=STACK_EPS, threads=th, record=False)
            n_cpu += 1
        dt = time.time() - c0
        cpu = {"value": round(n_cpu * n_tok / dt, 3), "unit": "tokens/s", "cores": th, "kind": "oracle",
               "sample": f"{n_cpu} passes of {n_tok} of the 32 tokens through all {NLAY} layers of the same "
                         f"stack (tokens are independent within a layer), {dt:.1f} s wall"}

    for d in dls:
        d.close()
    del dls, ws, wsl, x, x0, y, xin, rb
    torch.cuda.empty_cache()
    if args.copy_calibration:
        copy_calibration(torch)
    stream_ref = None if args.no_stream_reference else stream_reference(moe, torch)

    return {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s (% of peak), decode batch 1–256, 1 GPU",
        "value": round(T / (step_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": operand_dtype(fmt),
        "data": "synthetic",
        "hbm_gbps_expert_weights": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "hbm_frac_of_stream_read": round(gbps / stream_ref["gbps"], 4) if stream_ref else None,
        "stream_read": stream_ref,
        "config": {"workload": f"moe_stack_{args.workload}", "tokens": T, "layers": NLAY, "d_model": 2048,
                   "routed_experts": E, "top_k": K, "shared_experts": 1, "d_expert": 512, "weights": fmt,
                   "router_bias_zipf": cfg["zipf"], "rms_eps": STACK_EPS,
                   "touched_experts_mean": round(float(np.mean(touched)), 1),
                   "expert_weight_bytes_per_step": int(w_bytes), "router_bytes_per_step": NLAY * E * 2048 * 2,
                   "launch": ("hip_graph_replay" if graph_ms is not None else "plain") + (", persistent" if args.persistent else ""),
                   "plain_launch_ms_per_step": round(ms, 5), "graph_replay_ms": spread,
                   "per_layer_stage_ms": stage_means},
        "roofline": {"bound": "hbm", "kernel": "ffn_up_kernel (gate/up + SwiGLU), every layer of the stack",
                     "achieved": round(up_achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(up_achieved / HBM_PEAK_GBPS, 4),
                     "frac_of_stream_read": round(up_achieved / stream_ref["gbps"], 4) if stream_ref else None,
                     "traffic": None},
        "cpu_baseline": cpu,
    }


def head_row_bytes(fmt: str) -> int:
    """Stored bytes of one vocabulary row of 2048 columns."""
    return {"q4_1": 1024 + 64 * 4, "nvfp4": 1024 + 128, "bf16": 4096}[fmt]


def bench_head(args, moe, synth, torch, np):
    """Output-head GEMV: logits [T][V] of T tokens against a [V][2048] head.
    Steps rotate over --layers independently drawn heads (each 194 MB in q4_1,
    so that together they exceed the 256 MB last-level cache)."""
    cfg = synth.HEAD_CONFIGS[args.workload]
    T, fmt, V = cfg["T"], cfg["fmt"], cfg["V"]
    NL = max(1, args.layers)
    log(f"generating {NL} heads of {args.workload}")
    hosts = [synth.make_head(V, fmt, seed=s) for s in range(NL)]
    dms = [moe.DeviceMatrix(h) for h in hosts]
    x_bits = synth.make_x(T)
    x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    logits = torch.empty((T, V), dtype=torch.float32, device="cuda")
    stream = moe.current_stream()
    # algorithmic bytes of one launch: the head once, the tokens once, the logits once
    step_bytes = V * head_row_bytes(fmt) + (4 if fmt == "nvfp4" else 0) + T * 2048 * 2 + T * V * 4

    def step(i, on=None):
        dm = dms[i % NL]
        moe.moe_head_forward(x.data_ptr(), T, dm.qmat, moe.WFMT[fmt], V, 2048, logits.data_ptr(),
                             stream if on is None else on)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # per-launch durations: an event pair around each plain launch on the library's stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    log(f"timing {args.steps} plain launches")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        evs[i][0].record()
        step(args.warmup + i)
        evs[i][1].record()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(NL):
                step(i, on=moe.current_stream())
        n_full, n_rest = divmod(args.steps, NL)
        g_rest = None
        if n_rest:
            g_rest = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_rest):
                for i in range(n_rest):
                    step(i, on=moe.current_stream())
        for _ in range(max(1, args.warmup // NL)):
            g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(n_full):
            g.replay()
        if g_rest is not None:
            g_rest.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        log(f"graph replay: {graph_ms * 1e3:.1f} us per step; plain launches {ms * 1e3:.1f} us, "
            f"kernel {kern_ms * 1e3:.1f} us")
        del g, g_rest
    step_ms = graph_ms if graph_ms is not None else ms
    achieved = step_bytes / (kern_ms * 1e-3) / 1e9
    traffic = read_traffic(args.workload, "head")
    if args.copy_calibration:
        copy_calibration(torch)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        th = oracle.max_threads()
        log(f"cpu baseline: oracle on {th} threads, whole {T}-token steps for about 10 s")
        n_cpu, c0 = 0, time.time()
        while n_cpu < 1 or (time.time() - c0 < 10.0 and n_cpu < 64):
            oracle.head_logits(hosts[n_cpu % NL], x_bits, threads=th)
            n_cpu += 1
        dt = time.time() - c0
        cpu = {"value": round(n_cpu * T / dt, 3), "unit": "tokens/s", "cores": th, "kind": "oracle",
               "sample": f"{n_cpu} steps of the same workload (all {V} rows for the {T} tokens, fp64), "
                         f"{dt:.1f} s wall"}

    del dms, x, logits
    torch.cuda.empty_cache()
    stream_ref = None if args.no_stream_reference else stream_reference(moe, torch)
    return {
        "metric": "output-head tokens/s + achieved HBM GB/s (% of peak), 1 GPU",
        "value": round(T / (step_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{fmt} weights, {'bf16' if fmt == 'bf16' else 'f16'} operands, f32 accumulate",
        "data": "synthetic",
        "hbm_gbps": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
        "stream_read": stream_ref,
        "config": {"workload": f"output_head_{args.workload}", "tokens": T, "vocab": V, "d_model": 2048,
                   "weights": fmt, "head_instances": NL, "bytes_per_step": step_bytes,
                   "launch": "hip_graph_replay" if graph_ms is not None else "plain",
                   "plain_launch_ms_per_step": round(ms, 5), "kernel_ms": round(kern_ms, 5)},
        "roofline": {"bound": "hbm", "kernel": "head_kernel (T <= 4) / head_mf_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "frac_of_stream_read": round(achieved / stream_ref["gbps"], 4) if stream_ref else None,
                     "traffic": traffic},
        "cpu_baseline": cpu,
    }


def bench_attn(args, moe, synth, torch, np):
    """Decode attention: one new token for each of B sequences whose caches hold
    ctx positions (the token at position ctx - 1).  Steps rotate over --layers
    independently drawn caches (537 MB each at 32 x 8192), so that every step
    reads its keys and values from HBM."""
    cfg = synth.ATTN_CONFIGS[args.workload]
    B, ctx, window, rope = cfg["B"], cfg["ctx"], cfg["window"], cfg["rope"]
    NL = max(1, args.layers)
    HQ, HK, D = synth.ATTN_HQ, synth.ATTN_HK, synth.ATTN_D
    desc = moe.moe_attn_desc(window, int(rope), 10000.0, 1e-6)
    log(f"generating {NL} caches of {args.workload}")
    a = synth.make_attn(B, ctx, seed=0)

    def dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).cuda().view(torch.bfloat16)

    caches = []
    for i in range(NL):
        c = moe.AttnCache(B, ctx)
        if i == 0:
            c.load(a["k_cache"], a["v_cache"])
        else:  # further layers: a cheap device-side variant of the same draw
            c.k.copy_(caches[0].k.roll(i, dims=2))
            c.v_t.copy_(caches[0].v_t.roll(i, dims=2))
        caches.append(c)
    q, k, v = dev(a["q"]), dev(a["k"]), dev(a["v"])
    qg, kg = dev(a["q_gain"]), dev(a["k_gain"])
    sinks = torch.from_numpy(a["sinks"]).cuda()
    pos = torch.full((B,), ctx - 1, dtype=torch.int32, device="cuda")
    out = torch.empty((B, HQ, D), dtype=torch.bfloat16, device="cuda")
    ws = moe.alloc_workspace(moe.attn_workspace_size(desc, B, ctx))
    stream = moe.current_stream()
    span = min(window, ctx) if window else ctx
    # algorithmic bytes of one call: the attended keys and values once, the new
    # token's q, k, v and gains in, k' and v appended, out written
    step_bytes = B * HK * span * D * 2 * 2 + B * (HQ + 2 * HK) * D * 2 + 2 * D * 2 + B * HK * D * 2 * 2 + B * HQ * D * 2

    def step(i, on=None):
        c = caches[i % NL]
        moe.moe_attn_decode(desc, B, ctx, q.data_ptr(), k.data_ptr(), v.data_ptr(), qg.data_ptr(), kg.data_ptr(),
                            sinks.data_ptr(), pos.data_ptr(), c.k.data_ptr(), c.v_t.data_ptr(), ctx, out.data_ptr(),
                            ws.data_ptr(), ws.numel(), stream if on is None else on)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} plain calls")
    start.record()
    for i in range(args.steps):
        evs[i][0].record()
        step(args.warmup + i)
        evs[i][1].record()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    call_ms = float(np.mean([x.elapsed_time(y) for x, y in evs]))
    graph_ms = None
    if not args.no_graph:
        n_full, n_rest = divmod(args.steps, NL)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(NL):
                step(i, on=moe.current_stream())
        g_rest = None
        if n_rest:
            g_rest = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_rest):
                for i in range(n_rest):
                    step(i, on=moe.current_stream())
        for _ in range(max(1, args.warmup // NL)):
            g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(n_full):
            g.replay()
        if g_rest is not None:
            g_rest.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        log(f"graph replay: {graph_ms * 1e3:.1f} us per step; plain {ms * 1e3:.1f} us; call {call_ms * 1e3:.1f} us")
        del g, g_rest
    step_ms = graph_ms if graph_ms is not None else ms
    achieved = step_bytes / (call_ms * 1e-3) / 1e9
    if args.copy_calibration:
        copy_calibration(torch)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        th = oracle.max_threads()
        lens = np.full(B, ctx, np.int32)
        log(f"cpu baseline: oracle on {th} threads, whole steps for about 10 s")
        n_cpu, c0 = 0, time.time()
        while n_cpu < 1 or (time.time() - c0 < 10.0 and n_cpu < 64):
            qp, _ = oracle.attn_prep(a["q"], a["k"], a["q_gain"], a["k_gain"], lens - 1, rope)
            oracle.attn_decode(qp, a["k_cache"], a["v_cache"], lens, window, a["sinks"], threads=th)
            n_cpu += 1
        dt = time.time() - c0
        cpu = {"value": round(n_cpu * B / dt, 3), "unit": "tokens/s", "cores": th, "kind": "oracle",
               "sample": f"{n_cpu} steps of the same workload ({B} sequences, {span} attended positions each, "
                         f"fp64), {dt:.1f} s wall"}

    del caches, q, k, v, out, ws
    torch.cuda.empty_cache()
    stream_ref = None if args.no_stream_reference else stream_reference(moe, torch)
    return {
        "metric": "decode-attention tokens/s + achieved HBM GB/s (% of peak), 1 GPU",
        "value": round(B / (step_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 cache and operands, f32 accumulate and softmax",
        "data": "synthetic",
        "hbm_gbps": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
        "stream_read": stream_ref,
        "config": {"workload": f"decode_attention_{args.workload}", "sequences": B, "cached_positions": ctx,
                   "attended_positions": span, "window": window, "rope": rope, "q_heads": HQ, "kv_heads": HK,
                   "head_dim": D, "cache_instances": NL, "bytes_per_step": step_bytes,
                   "launch": "hip_graph_replay" if graph_ms is not None else "plain",
                   "plain_launch_ms_per_step": round(ms, 5), "call_ms": round(call_ms, 5)},
        "roofline": {"bound": "hbm", "kernel": "attention call (attn_decode_kernel + attn_combine_kernel)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "frac_of_stream_read": round(achieved / stream_ref["gbps"], 4) if stream_ref else None,
                     "traffic": read_traffic(args.workload, "attn")},
        "cpu_baseline": cpu,
    }


def bench_mfma_rate(args, moe, torch):
    """Attainable matrix-core rate per instruction kind (moe_mfma_rate): the
    reference against which the tile path's matrix-core utilisation is read."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")
    stream = moe.current_stream()
    grid, iters, reps = 2 * n_cu, 4096, max(3, args.steps // 20)
    rates = {}
    for kind, (name, flop) in moe.MFMA_KINDS.items():
        moe.moe_mfma_rate(kind, iters, grid, sink.data_ptr(), stream)  # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            moe.moe_mfma_rate(kind, iters, grid, sink.data_ptr(), stream)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tflops = grid * 4 * iters * 4 * flop / (ms * 1e-3) / 1e12
        rates[name] = {"tflops": round(tflops, 1), "ms_per_launch": round(ms, 4)}
        log(f"{name}: {tflops:.1f} TFLOP/s ({ms:.3f} ms per launch)")
    f16 = rates[moe.MFMA_KINDS[0][0]]["tflops"]
    for v in rates.values():
        v["vs_f16"] = round(v["tflops"] / f16, 3)
    return {"metric": "matrix-core instruction rate (measurement helper, not the layer)", "unit": "TFLOP/s",
            "workgroups": grid, "waves_per_simd": 2, "instructions_per_wave": 4 * iters, "rates": rates,
            "published_dense_peaks_tflops": {"f16/bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}}


def bench_read_patterns(args, moe, torch):
    """HBM read rate per access pattern (moe_read_pattern): a 1 GiB buffer read
    in regions of rows of 1 KB (4-bit rows of 2048) and 4 KB (bf16 rows), on
    2 and 4 workgroups per CU, best of the two, 5 launches each."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(3)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    stream = moe.current_stream()
    res = {}
    for row_bytes in (1024, 4096):
        for p, (name, rows) in moe.READ_PATTERNS.items():
            best = None
            for grid in (2 * n_cu, 4 * n_cu):
                moe.moe_read_pattern(p, src.data_ptr(), nbytes, row_bytes, grid, sink.data_ptr(), stream)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(5):
                    moe.moe_read_pattern(p, src.data_ptr(), nbytes, row_bytes, grid, sink.data_ptr(), stream)
                e1.record()
                torch.cuda.synchronize()
                gbps = nbytes * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
                best = max(best or 0.0, gbps)
            res[f"{name}, rows of {row_bytes} B"] = round(best, 1)
            log(f"pattern {p} ({name}), rows of {row_bytes} B: {best:.0f} GB/s")
    del src
    return {"metric": "HBM read rate per load-instruction access pattern (measurement helper, not the layer)",
            "unit": "GB/s", "bytes": nbytes, "loads_in_flight_per_lane": 8, "rates": res}


def bench_release_cost(args, moe, torch):
    """Cost of agent-scope releases at the end of every workgroup
    (moe_release_cost): us per launch for each mode, grid and data size."""
    stream = moe.current_stream()
    grids, pts = (512, 2048, 8192), (4, 16)
    data = torch.zeros(max(grids) * 256 * max(pts), dtype=torch.float32, device="cuda")
    ctr = torch.zeros(4096, dtype=torch.int32, device="cuda")
    res = []
    for grid in grids:
        for pt in pts:
            row = {"workgroups": grid, "kib_written_per_workgroup": pt}
            for mode, name in moe.RELEASE_MODES.items():
                moe.moe_release_cost(mode, data.data_ptr(), ctr.data_ptr(), grid, pt, stream)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(20):
                    moe.moe_release_cost(mode, data.data_ptr(), ctr.data_ptr(), grid, pt, stream)
                e1.record()
                torch.cuda.synchronize()
                row[name] = round(e0.elapsed_time(e1) * 1e3 / 20, 2)
            log(f"{row}")
            res.append(row)
    return {"metric": "agent-scope release cost (measurement helper, not the layer)", "unit": "us per launch",
            "table": res}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_t64_q4_1")
    ap.add_argument("--layers", type=int, default=8, help="layer instances the steps rotate over (single layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time plain launches instead of HIP-graph replays")
    ap.add_argument("--no-sweep", action="store_true", help="skip the token-count sweep")
    ap.add_argument("--no-stream-reference", action="store_true", help="skip the 4 GiB streaming-read reference")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--persistent", action="store_true",
                    help="time the persistent decode path (moe_layer_forward_persistent / moe_stack_forward_persistent);"
                         " the roofline's per-kernel timing stays on the kernel chain")
    ap.add_argument("--mfma-rate", action="store_true",
                    help="only time the matrix-core rate helper per instruction kind (f16, bf16, fp8, scaled fp4)")
    ap.add_argument("--read-patterns", action="store_true",
                    help="only time the HBM read rate of each load-instruction access pattern")
    ap.add_argument("--release-cost", action="store_true",
                    help="only time agent-scope releases at the end of every workgroup")
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
    if args.mfma_rate:
        out = bench_mfma_rate(args, moe, torch)
    elif args.read_patterns:
        out = bench_read_patterns(args, moe, torch)
    elif args.release_cost:
        out = bench_release_cost(args, moe, torch)
    elif args.workload in synth.HEAD_CONFIGS:
        out = bench_head(args, moe, synth, torch, np)
    elif args.workload in synth.ATTN_CONFIGS:
        out = bench_attn(args, moe, synth, torch, np)
    elif args.workload not in synth.CONFIGS:
        print(f"unknown workload {args.workload}; one of "
              f"{sorted(synth.CONFIGS) + sorted(synth.HEAD_CONFIGS) + sorted(synth.ATTN_CONFIGS)}",
              file=sys.stderr)
        return 2
    elif synth.CONFIGS[args.workload]["layers"] == 1:
        out = bench_layer(args, moe, synth, torch, np)
    else:
        out = bench_stack(args, moe, synth, torch, np)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
