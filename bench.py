#!/usr/bin/env python3
"""Throughput of causal kernelized linear attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload long] [--gpus 1]

A step is one la_forward call over the whole workload batch (all three
kernels: per-span state, span scan, chunked output).  Inputs are seeded
synthetic tensors already resident in HBM when the timed region starts;
three copies of the inputs and outputs are used in turn, so that no step
finds its data in the 256 MB memory-side cache left by the step before.  The
timed region is exactly K steps bracketed by device synchronisation; the
dominant kernel's duration comes from HIP events that the library records on
its stream around that kernel during those same steps.

Before timing, after the W warm-up steps, untimed steps continue for a fixed
wall time (--settle, 0.3 s by default): the GPU's clock and power control
takes about 10 ms of sustained load to reach its steady state, and a step
timed before that runs up to 25 % slower.

One JSON line is printed with the metric, the roofline of the dominant kernel
(the output kernel) and of the whole step, and the fp64 CPU oracle timed on
this host's cores (one worker process per core, up to 16, each running the
oracle on whole (batch, head) pairs) on the same workload.

Workloads (names from kernelized_linear_attention_elu_amd.synth.WORKLOADS):
long (default: B1 H32 N32768 d64 bf16 causal), prefill, wide, plus
``decode`` (one decode step for 256 sequences x 32 heads, d = 128) and
``feature`` (standalone ELU+1 feature map over the long workload's Q).
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal LA prefill tokens/s at N=32k,d=64 bf16; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
KERNEL_NAMES = ("la_state_kernel", "la_scan_kernel", "la_output_kernel")
FAVOR_KERNEL_NAMES = ("la_state_favor_kernel", "la_scan_kernel", "la_output_favor_kernel")
GLA_KERNEL_NAMES = ("la_state_kernel_gla", "la_scan_kernel", "la_output_kernel_gla")
BACKWARD_KERNEL_NAMES = ("la_state_kernel", "la_scan_kernel", "la_bwd_dq_kernel", "la_suffix_scan_kernel",
                         "la_bwd_dkv_kernel")
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "kernelized_linear_attention_elu_amd", "csrc")
ROTATE = 3                     # input/output copies used in turn by the prefill bench
SETTLE_S = 0.3                 # untimed run after the warm-up steps (clock/power steady state)


def settle(torch, run, seconds):
    """Keep calling run(i) (untimed) until `seconds` of wall time have passed,
    synchronising every 16 calls; returns the number of calls."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            run(i)
            i += 1
        torch.cuda.synchronize()
    return i


def source_hash():
    """sha256 over the HIP sources: counter figures taken for other sources
    are stale and are not reported."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload, kernel):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current sources."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path, encoding="utf-8") as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("source_hash") != source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="long",
                   choices=["long", "prefill", "wide", "favor", "decode", "feature", "copy"])
    p.add_argument("--noncausal", action="store_true", help="non-causal prefill")
    p.add_argument("--decay", action="store_true",
                   help="causal prefill with a fixed per-head decay (RetNet form, la_forward_decay)")
    p.add_argument("--gated", action="store_true",
                   help="causal prefill with a per-token scalar gate (SSD scalar-decay form, la_forward_gated)")
    p.add_argument("--backward", action="store_true",
                   help="the backward pass of the causal prefill (la_backward: dQ, dK, dV for an upstream dO)")
    p.add_argument("--gla", action="store_true",
                   help="causal prefill with a per-token, per-key-channel gate (GLA form, la_forward_gla)")
    p.add_argument("--chunk", type=int, default=None,
                   help="chunk size (default: the workload's, 0 = the library's choice)")
    p.add_argument("--settle", type=float, default=SETTLE_S,
                   help="seconds of untimed steps after the warm-up steps (clock/power steady state)")
    p.add_argument("--span-tokens", type=int, default=0,
                   help="span length of the chunkwise prefill (a multiple of the chunk; 0: the library's choice)")
    p.add_argument("--precise", action="store_true",
                   help="FAVOR+ workload: the precise form (omega hi + lo in the output pass)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args(argv)


def cpu_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def _oracle_head(q, k, v, a, alpha, causal=True, phi="elu1", omega=None, gamma=None):
    """The fp64 oracle on one (batch, head): the token recurrence (decayed,
    gated or per-channel gated when given), or the reassociated non-causal
    form."""
    from oracle import linear_attention as ora
    from oracle import decay as dec
    from oracle import gated as gat
    from oracle import gla
    if alpha is not None:
        return gla.recurrent_gla(q, k, v, alpha, phi=phi)[0]
    if a is not None:
        return gat.recurrent_gated(q, k, v, a, phi=phi)[0]
    if gamma is not None:
        return dec.recurrent_decay(q, k, v, gamma, phi=phi)[0]
    if causal:
        return ora.recurrent_attention(q, k, v, phi=phi, omega=omega)[0]
    return ora.noncausal_attention(q, k, v, phi=phi, omega=omega)[0]


def time_oracle_prefill(q, k, v, causal, phi="elu1", omega=None, gamma=None, log_a=None, log_a_ch=None):
    """fp64 oracle over every (batch, head) of the workload in the worker pool
    (oracle/heads.py); returns (seconds, heads, workers)."""
    from oracle import heads
    import numpy as np
    a = np.exp(log_a.astype("float64")) if log_a is not None else None
    alpha = np.maximum(np.exp(log_a_ch.astype("float64")), 2.0 ** -14) if log_a_ch is not None else None
    t0 = time.perf_counter()
    heads.map_heads(_oracle_head, q, k, v, a, alpha, causal=causal, phi=phi, omega=omega,
                    head_kw=lambda b, h: {"gamma": float(gamma[h]) if gamma is not None else None})
    wall = time.perf_counter() - t0
    return wall, q.shape[0] * q.shape[1], heads.processes()


def bench_prefill(args, torch, la, synth):
    from kernelized_linear_attention_elu_amd import hostio
    w = synth.WORKLOADS[args.workload]
    if args.span_tokens:
        la.set_span_tokens(args.span_tokens)
    if args.chunk is not None:
        w = dataclasses.replace(w, chunk=args.chunk)
    causal = not args.noncausal
    if (args.decay or args.gated or args.gla) and (not causal or w.phi == "favor"):
        raise SystemExit("--decay / --gated / --gla: causal pointwise-feature workloads only")
    if args.decay + args.gated + args.gla > 1:
        raise SystemExit("--decay, --gated and --gla exclude each other")
    if args.gla and w.d == 128 and args.chunk is None:
        w = dataclasses.replace(w, chunk=32)   # the per-channel gated kernels take chunks up to 32 at d = 128
    dev = torch.device("cuda:0")
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)
    gamma = synth.decay_gammas(w.H) if args.decay else None
    log_a = synth.draw_log_gates(w.B, w.H, w.N) if args.gated else None
    log_a_ch = synth.draw_log_gates_ch(w.B, w.H, w.N, w.r) if args.gla else None

    def to_dev(x):
        return hostio.upload_bf16_bits(synth.bf16_bits(x), dev)

    # ROTATE copies of the inputs and outputs, used in turn, so that no step
    # finds its data in the 256 MB memory-side cache left by the previous
    # step: every step streams its inputs from HBM
    Q0, K0, V0 = to_dev(q), to_dev(k), to_dev(v)
    sets = [(Q0, K0, V0)] + [(Q0.clone(), K0.clone(), V0.clone()) for _ in range(ROTATE - 1)]
    outs = [torch.empty((w.B, w.H, w.N, w.dv), dtype=torch.bfloat16, device=dev) for _ in range(ROTATE)]
    omega = synth.draw_omega(w.r, w.d) if w.phi == "favor" else None
    lib_phi = "favor_precise" if (w.phi == "favor" and args.precise) else w.phi
    om_dev = hostio.upload_f32(omega, dev) if omega is not None else None
    gamma_dev = hostio.upload_f32(gamma, dev) if gamma is not None else None
    gates = gates_ch = None
    if log_a is not None:
        g0 = hostio.upload_f32(log_a, dev)
        gates = [g0] + [g0.clone() for _ in range(ROTATE - 1)]
    if log_a_ch is not None:
        g0 = hostio.upload_f32(log_a_ch, dev)
        gates_ch = [g0] + [g0.clone() for _ in range(ROTATE - 1)]
    ws = torch.empty(la.workspace_bytes(w.B, w.H, w.N, w.d, w.dv, io=w.io, phi=lib_phi, r=w.r, causal=causal,
                                        chunk=w.chunk, gated=log_a is not None, gla=log_a_ch is not None),
                     dtype=torch.uint8, device=dev)

    def step(i, events=None):
        Q, K, V = sets[i % ROTATE]
        la.forward(Q, K, V, phi=lib_phi, omega=om_dev, causal=causal, chunk=w.chunk, out=outs[i % ROTATE],
                   workspace=ws, events=events, gamma=gamma_dev,
                   log_gate=gates[i % ROTATE] if gates is not None else None,
                   log_gate_ch=gates_ch[i % ROTATE] if gates_ch is not None else None)

    for i in range(args.warmup):
        step(i)
    settled = settle(torch, step, args.settle)
    nk = la.LA_FORWARD_KERNELS
    evs = [[la.event_create() for _ in range(2 * nk)] for _ in range(args.steps)]
    # timed region: exactly K steps; two HIP events per step, recorded by the
    # library on its stream around the dominant (output) kernel, give that
    # kernel's duration live
    live = [[None] * (2 * nk - 2) + e[2 * nk - 2:] for e in evs]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, live[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    out_live_ms = sum(la.event_elapsed_ms(e[2 * nk - 2], e[2 * nk - 1]) for e in evs) / args.steps
    # breakdown of the whole step: K more steps with events around every
    # kernel (these add gaps between kernels, so they are kept out of the
    # timed region)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    kern_ms = [0.0] * la.LA_FORWARD_KERNELS
    for e in evs:
        for j in range(la.LA_FORWARD_KERNELS):
            kern_ms[j] += la.event_elapsed_ms(e[2 * j], e[2 * j + 1]) / args.steps
    for e in evs:
        for x in e:
            la.event_destroy(x)

    ms = (t1 - t0) * 1e3 / args.steps
    token_heads = w.B * w.H * w.N
    alg_bytes = token_heads * (2 * w.d + 2 * w.dv) * 2          # read Q, K, V, write O (bf16)
    if log_a is not None:
        alg_bytes += token_heads * 4                             # read the fp32 log gates
    if log_a_ch is not None:
        alg_bytes += token_heads * 4 * w.r                       # read the fp32 per-channel log gates
    # features (FAVOR+: two d x r projections), state build + read-out
    # (4 r dv), intra-chunk products over full C x C tiles
    feat_flops = 2 * 2 * w.d * w.r if w.phi == "favor" else 0
    alg_flops = token_heads * (feat_flops + 4 * w.r * w.dv + (2 * w.chunk * (w.r + w.dv) if causal else 0))
    out_ms = out_live_ms
    n_span, single_pass = la.forward_config(w.B, w.H, w.N, w.d, w.dv, io=w.io, phi=lib_phi, r=w.r, causal=causal,
                                            chunk=w.chunk, decay=gamma is not None, gated=log_a is not None,
                                            gla=log_a_ch is not None)
    names = (FAVOR_KERNEL_NAMES if w.phi == "favor" else GLA_KERNEL_NAMES if log_a_ch is not None
             else KERNEL_NAMES)
    out_kernel = names[2]
    # the decayed and gated variants of la_output_kernel are other kernels:
    # their counter figures are kept under their own workload tag
    mode = ("_decay" if gamma is not None else "_gated" if log_a is not None
            else "_precise" if lib_phi == "favor_precise" else "")
    traffic = read_traffic(args.workload + ("" if causal else "_noncausal") + mode, out_kernel)
    if w.phi == "favor":
        # the output kernel's own work: phi(Q) and phi(K) projections, the
        # read-out and the state carry (2 r dv each), the intra-chunk products
        out_flops = token_heads * (2 * 2 * w.d * w.r + 2 * 2 * w.r * w.dv
                                   + (2 * w.chunk * (w.r + w.dv) if causal else 0))
        achieved = out_flops / (out_ms * 1e-3) / 1e12
        roof = {"kernel": out_kernel, "bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS, "traffic": traffic,
                "scope": "dominant kernel only; the whole call: path_roofline"}
    else:
        # the output kernel reads Q, K, V and writes O (causal); non-causal it
        # reads Q and writes O only
        out_bytes = alg_bytes if causal else token_heads * (w.d + w.dv) * 2  # (gated: with the gates)
        achieved = out_bytes / (out_ms * 1e-3) / 1e9
        roof = {"kernel": out_kernel, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "scope": "dominant kernel only; the whole call: path_roofline"}
    step_gbs = alg_bytes / (ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": w.B * w.N / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name} prefill B{w.B} H{w.H} N{w.N} d{w.d} dv{w.dv} bf16 I/O, fp32 state, "
                        f"phi={'FAVOR+ r=%d' % w.r if w.phi == 'favor' else 'elu+1'}"
                        f"{' (precise form)' if lib_phi == 'favor_precise' else ''}, "
                        f"{'causal' if causal else 'non-causal'}, chunk {w.chunk}"
                        + (", per-head decay gamma_h = 1 - 2^-(5 + 7h/(H-1)) (RetNet form)" if gamma is not None else "")
                        + (", per-token gates log a = -dt A_h, dt log-uniform [1e-3, 1e-1], A_h = 1 + 15h/(H-1)"
                           " (SSD scalar-decay form)" if log_a is not None else "")
                        + (", per-token per-key-channel gates sigmoid(x)^(1/16), x ~ N(0, 4) (GLA form)"
                           if log_a_ch is not None else ""),
            "B": w.B, "H": w.H, "N": w.N, "d": w.d, "dv": w.dv, "r": w.r, "chunk": w.chunk, "causal": causal,
            "phi": w.phi, "accumulate": "fp32", "decay": gamma is not None, "gated": log_a is not None,
            "gla": log_a_ch is not None,
        },
        "roofline": roof,
        "path_roofline": {
            "scope": "whole call: every kernel of the step, algorithmic bytes over the step time",
            "bound": "hbm",
            "alg_bytes": alg_bytes,
            "alg_flops": alg_flops,
            "achieved_gbs": step_gbs,
            "frac": step_gbs / HBM_PEAK_GBS,
            "mfma_frac": alg_flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        },
        "kernels_us": {n: t * 1e3 for n, t in zip(names, kern_ms) if n},
        "dominant_kernel_us_live": out_live_ms * 1e3,
        "path": {"single_pass": single_pass, "spans_per_head": n_span},
        "settle": {"seconds": args.settle, "untimed_steps": settled},
    }
    if not args.no_cpu_baseline:
        wall, h, cores = time_oracle_prefill(q, k, v, causal, phi=w.phi, omega=omega, gamma=gamma,
                                             log_a=log_a, log_a_ch=log_a_ch)
        form = (('per-channel gated token recurrence' if log_a_ch is not None else 'gated token recurrence'
                 if log_a is not None else 'decayed token recurrence' if gamma is not None else 'token recurrence')
                if causal else 'reassociated form')
        res["cpu_baseline"] = {
            "value": w.B * w.N / wall,
            "unit": "tokens/s",
            "cores": cores,
            "kind": "oracle",
            "sample": f"the whole job: fp64 {form} over all {h} heads x {w.N} tokens ({wall:.1f} s), "
                      f"one (batch, head) at a time per worker process",
            "cpu": cpu_info(),
        }
    return res


def bench_backward(args, torch, la, synth):
    """One step = la_backward over the workload: the forward span states and
    their scan, the dQ pass, the reverse scan, the dK/dV pass, with Q, K, V,
    O (the library's forward output) and dO resident in HBM."""
    from kernelized_linear_attention_elu_amd import hostio
    import numpy as np
    w = synth.WORKLOADS[args.workload]
    if w.phi == "favor" or w.d not in (64, 128) or args.noncausal:
        raise SystemExit("--backward: causal, d = 64 or 128, pointwise feature maps")
    if args.span_tokens:
        la.set_span_tokens(args.span_tokens)
    dev = torch.device("cuda:0")
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)
    rng = np.random.default_rng(91)
    dO = synth.round_to_io(rng.standard_normal((w.B, w.H, w.N, w.dv), dtype=np.float32), "bf16")

    def to_dev(x):
        return hostio.upload_bf16_bits(synth.bf16_bits(x), dev)

    Q0, K0, V0, G0 = to_dev(q), to_dev(k), to_dev(v), to_dev(dO)
    O0 = la.forward(Q0, K0, V0, phi=w.phi)
    sets = [(Q0, K0, V0, O0, G0)] + [tuple(t.clone() for t in (Q0, K0, V0, O0, G0)) for _ in range(ROTATE - 1)]
    outs = [(torch.empty_like(Q0), torch.empty_like(K0), torch.empty_like(V0)) for _ in range(ROTATE)]
    ws = torch.empty(int(la.load_library().la_backward_workspace_bytes(w.B, w.H, w.N, w.d, w.dv, la.LA_BF16,
                                                                        la.PHI[w.phi], 0, 64)),
                     dtype=torch.uint8, device=dev)

    def step(i, events=None):
        Q, K, V, O, G = sets[i % ROTATE]
        la.backward(Q, K, V, O, G, phi=w.phi, out=outs[i % ROTATE], workspace=ws, events=events)

    for i in range(args.warmup):
        step(i)
    settled = settle(torch, step, args.settle)
    nk = la.LA_BACKWARD_KERNELS
    evs = [[la.event_create() for _ in range(2 * nk)] for _ in range(args.steps)]
    live = [[None] * (2 * nk - 2) + e[2 * nk - 2:] for e in evs]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, live[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    last_live_ms = sum(la.event_elapsed_ms(e[2 * nk - 2], e[2 * nk - 1]) for e in evs) / args.steps
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    kern_ms = [0.0] * nk
    for e in evs:
        for j in range(nk):
            kern_ms[j] += la.event_elapsed_ms(e[2 * j], e[2 * j + 1]) / args.steps
    for e in evs:
        for x in e:
            la.event_destroy(x)
    ms = (t1 - t0) * 1e3 / args.steps
    token_heads = w.B * w.H * w.N
    # the dK/dV pass (timed live, the last kernel of the step) reads Q, K, V,
    # dO and (D_i, h_i), writes dK, dV
    pass_b_bytes = token_heads * ((3 * w.d + w.dv) * 2 + 8 + (w.d + w.dv) * 2)
    achieved = pass_b_bytes / (last_live_ms * 1e-3) / 1e9
    n_span = int(ctypes_config(la, w))
    step_bytes = token_heads * ((w.d + w.dv) * 2                     # forward span states read K, V (+ scan)
                                + ((2 * w.d + 3 * w.dv) * 2 + w.d * 2 + 8)   # dQ pass
                                + ((2 * w.d + 2 * w.dv) * 2 + 8 + (w.d + w.dv) * 2))  # dK/dV pass
    res = {
        "metric": "causal LA backward tokens/s at N=32k,d=64 bf16 (dQ, dK, dV)",
        "value": w.B * w.N / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name} backward B{w.B} H{w.H} N{w.N} d{w.d} dv{w.dv} bf16 I/O, fp32 states, "
                        f"phi=elu+1, causal, chunk 64, dO ~ N(0, 1)",
            "B": w.B, "H": w.H, "N": w.N, "d": w.d, "dv": w.dv, "chunk": 64, "phi": w.phi, "backward": True,
        },
        "roofline": {"kernel": "la_bwd_dkv_kernel", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": read_traffic(args.workload + "_backward", "la_bwd_dkv_kernel"),
                     "scope": "dominant kernel only; the whole call: path_roofline"},
        "path_roofline": {"scope": "whole call", "bound": "hbm", "alg_bytes": step_bytes,
                          "achieved_gbs": step_bytes / (ms * 1e-3) / 1e9,
                          "frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "kernels_us": {n: t * 1e3 for n, t in zip(BACKWARD_KERNEL_NAMES, kern_ms)},
        "dominant_kernel_us_live": last_live_ms * 1e3,
        "path": {"spans_per_head": n_span},
        "settle": {"seconds": args.settle, "untimed_steps": settled},
    }
    if not args.no_cpu_baseline:
        from oracle import heads
        t_a = time.perf_counter()
        heads.map_heads(_grad_head, q, k, v, dO)
        wall = time.perf_counter() - t_a
        res["cpu_baseline"] = {
            "value": w.B * w.N / wall, "unit": "tokens/s", "cores": heads.processes(),
            "kind": "oracle",
            "sample": f"the whole job: fp64 prefix/suffix-state gradient loops over all {w.B * w.H} heads x {w.N} "
                      f"tokens ({wall:.1f} s), one (batch, head) at a time per worker process",
            "cpu": cpu_info(),
        }
    return res


def _grad_head(q, k, v, dO):
    """dQ, dK, dV of one (batch, head) from the fp64 gradient oracle."""
    from oracle import backward as bwd
    return bwd.grad_rows(q, k, v, dO, range(q.shape[-2]))


def ctypes_config(la, w):
    import ctypes
    n = ctypes.c_int()
    la.load_library().la_backward_config(w.B, w.H, w.N, w.d, w.dv, la.LA_BF16, la.PHI[w.phi], 0, 64,
                                         ctypes.byref(n))
    return n.value


def bench_decode(args, torch, la, synth):
    from kernelized_linear_attention_elu_amd import hostio
    import numpy as np
    dw = synth.DECODE_WORKLOAD
    n, H, d, dv, T = dw["n_seq"], dw["H"], dw["d"], dw["dv"], dw["history"]
    dev = torch.device("cuda:0")

    def to_dev(x):
        return hostio.upload_bf16_bits(synth.bf16_bits(x), dev)

    kh, vh = synth.draw_decode_history(n, H, T, d, dv)
    # the state comes from a prefill of the history through the library itself
    _, S, z = la.forward(to_dev(np.zeros_like(kh)), to_dev(kh), to_dev(vh), return_state=True)
    q, k, v = (to_dev(x) for x in synth.draw_decode_token(n, H, d, dv))
    o = torch.empty((n, H, dv), dtype=torch.bfloat16, device=dev)
    for _ in range(args.warmup):
        la.decode_step(S, z, q, k, v, out=o)
    settled = settle(torch, lambda i: la.decode_step(S, z, q, k, v, out=o), args.settle)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        la.decode_step(S, z, q, k, v, out=o)
    end.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    kern_ms = start.elapsed_time(end) / args.steps
    per_head = d * dv * 4 * 2 + d * 4 * 2 + (2 * d + 2 * dv) * 2
    alg_bytes = n * H * per_head
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "decode steps/s (256 sequences x 32 heads, d=dv=128, fp32 state, bf16 tokens)",
        "value": n / (ms * 1e-3),
        "unit": "sequence-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"decode step {n} seq x {H} heads d{d} dv{dv}, state from a {T}-token prefill",
                   "n_seq": n, "H": H, "d": d, "dv": dv},
        "roofline": {"kernel": "la_decode_kernel", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": read_traffic("decode", "la_decode_kernel")},
        "settle": {"seconds": args.settle, "untimed_steps": settled},
    }
    return res


def bench_feature(args, torch, la, synth):
    from kernelized_linear_attention_elu_amd import hostio
    import numpy as np
    w = synth.WORKLOADS["long"]
    dev = torch.device("cuda:0")
    q, _, _ = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io="bf16")
    X = hostio.upload_bf16_bits(synth.bf16_bits(q), dev)
    del q
    Y = torch.empty(tuple(X.shape), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        la.feature_map(X, out=Y)
    settled = settle(torch, lambda i: la.feature_map(X, out=Y), args.settle)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        la.feature_map(X, out=Y)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    alg_bytes = X.numel() * 2 + Y.numel() * 4
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    return {
        "metric": "ELU+1 feature map rows/s (bf16 in, fp32 out)",
        "value": X.numel() // w.d / (ms * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"phi over Q of the long prefill ({X.numel() // w.d} rows x {w.d})"},
        "roofline": {"kernel": "la_phi_pointwise_kernel", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": read_traffic("feature", "la_phi_pointwise_kernel")},
        "settle": {"seconds": args.settle, "untimed_steps": settled},
    }


def bench_copy(args, torch):
    """Plain device copy of a known size: the reference for scaling the HBM
    byte counters of the other kernels."""
    n = 256 * 1024 * 1024
    a = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(args.warmup):
        b.copy_(a)
    settled = settle(torch, lambda i: b.copy_(a), args.settle)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        b.copy_(a)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    return {"metric": "device copy GB/s (read + write)", "value": 2 * n / (ms * 1e-3) / 1e9, "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
            "data": "synthetic", "config": {"workload": f"copy of {n} bytes", "bytes_read": n, "bytes_written": n},
            "settle": {"seconds": args.settle, "untimed_steps": settled}}


def main(argv=None):
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (heads shard across GPUs "
              "with no exchange; the sequence would shard with one exchange of span states); "
              "run with --gpus 1", file=sys.stderr)
        return 2
    if not args.no_cpu_baseline and args.workload not in ("copy", "decode", "feature"):
        # the oracle's worker processes are forked before anything touches
        # the GPU, so that none of them inherits GPU state
        from oracle import heads
        heads.start()
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    import kernelized_linear_attention_elu_amd as la
    from kernelized_linear_attention_elu_amd import synth
    if args.workload == "copy":
        res = bench_copy(args, torch)
    else:
        la.load_library()
        if args.workload == "decode":
            res = bench_decode(args, torch, la, synth)
        elif args.workload == "feature":
            res = bench_feature(args, torch, la, synth)
        elif args.backward:
            res = bench_backward(args, torch, la, synth)
        else:
            res = bench_prefill(args, torch, la, synth)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
