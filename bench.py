#!/usr/bin/env python3
"""MoE-layer forward benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--also NAME,...] [--graph]

A step is one full layer call (router GEMM, top-k, dispatch, expert GEMMs / weight streaming,
shared expert, combine) over one batch of seeded synthetic tokens already resident in HBM. A
workload named "<config>+backward" times the layer's backward pass instead (reported under
'also'), with fp32 gradients, and beside it the same pass writing the expert weight gradients
in bf16.
Prints one JSON line: tokens/s, the dominant kernel's roofline fraction (HIP events around that
kernel's launches during the timed region, against algorithmic bytes or flops), and the
double-precision oracle timed on a bounded token sample on the host as the CPU baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s, Nano shape (T=64 decode, T=8192 prefill); % roofline"
PEAK_HBM = 8.0e12            # B/s, MI355X HBM3E
PEAK_MFMA = {"bf16": 2.5e15, "fp8": 5.0e15, "f32": 157.3e12}   # dense FLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="nano_decode_bf16")
    ap.add_argument("--also", default="nano_prefill_bf16,latent_bf16,nano_fp8,tiny_f32,"
                                      "latent_decode_bf16,nano_fp8_decode,"
                                      "nano_mxfp4_decode,nano_mxfp8_decode,latent_mxfp4_decode,"
                                      "latent_fp8_decode,nano_prefill_bf16+backward,"
                                      "latent_bf16+backward",
                    help="comma-separated extra workloads reported under 'also' ('' for none)")
    ap.add_argument("--path", default="auto", choices=["auto", "grouped", "stream"])
    ap.add_argument("--graph", action="store_true", help="replay the step as a captured graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-wgrad-bf16", action="store_true",
                    help="backward workloads: skip the extra timing of the bf16 weight-gradient "
                         "pass (counter runs then see the fp32 pass alone)")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0: auto)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one device copy of MIB MiB (a known-size reference for "
                         "hardware byte counters)")
    return ap.parse_args()


# ------------------------------------------------------------------ algorithmic work per launch

def work_of(name, cfg, counts, stream=False):
    """(flops, bytes) one launch of trace span `name` must do for layer `cfg`; expert weights of
    the touched experts counted once, activations counted once in and once out."""
    T, H, E, k, I, Is, L = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.latent
    D, P = cfg.D, cfg.T * cfg.k
    ea = 4 if cfg.act_dtype == "f32" else 2
    # weight bytes per element; 8-bit and 4-bit experts meet e4m3 token rows
    ew = {"f32": 4, "bf16": 2, "e4m3": 1, "mxfp8": 1, "mxfp4": 0.5}[cfg.expert_dtype]
    narrow = cfg.expert_dtype in ("e4m3", "mxfp4", "mxfp8")
    mx = cfg.expert_dtype in ("mxfp4", "mxfp8")
    touched = int(np.count_nonzero(counts))

    def scales(rows, K):   # e4m3: fp32 per output channel; MX: one E8M0 byte per 32 along K
        if mx:
            return touched * rows * (K // 32)
        return touched * rows * 4 if narrow else 0

    role = name.split(":")[1]
    if role.startswith("bwd_") or role in ("pairs", "gates", "du", "dx", "dW_r"):
        return backward_work(role, cfg, touched)
    if role == "router":
        return 2 * T * E * H, T * H * ea + E * H * ea + T * E * 4
    # stream launches: routed projection, plus the shared expert's on a bf16 plain layer
    sh = bool(Is and not L and not narrow)
    if role == "up":
        f = 2 * P * I * D + (2 * T * Is * H if sh else 0)
        b = touched * I * D * ew + scales(I, D) + T * D * (1 if narrow else ea) + P * I * 2
        if sh:
            b += Is * H * ea + T * Is * 2
        return f, int(b)
    if role == "down":     # fp32 outputs
        f = 2 * P * D * I + (2 * T * H * Is if sh else 0)
        b = touched * D * I * ew + scales(D, I) + P * I * (1 if narrow else 2) + P * D * 4
        if sh:
            b += H * Is * ea + T * Is * 2 + T * H * 4
        return f, int(b)
    if role == "routed_up":
        return 2 * P * I * D, int(touched * I * D * ew + scales(I, D) +
                                  T * D * (1 if narrow else ea) + P * I * 2)
    if role == "routed_down":
        h_in = P * I * (1 if narrow else 2)
        return 2 * P * D * I, int(touched * D * I * ew + scales(D, I) + h_in +
                                  P * D * (4 if stream else ea))
    if role == "shared_up":
        return 2 * T * Is * H, Is * H * ea + T * H * ea + T * Is * ea
    if role == "shared_down":  # fp32 output
        return 2 * T * H * Is, H * Is * ea + T * Is * ea + T * H * 4
    if role == "latent_in":
        return 2 * T * L * H, L * H * ea + T * H * ea + T * L * ea
    if role == "latent_out":
        f = 2 * T * H * L + (2 * T * H * Is if Is else 0)
        return f, H * L * ea + T * L * ea + T * H * ea + (H * Is * ea + T * Is * ea if Is else 0)
    if role in ("y", "z"):
        yb = 4 if stream else ea
        s_in = T * H * 4 if (Is and not L and role == "y") else 0
        return 2 * P * D, P * D * yb + s_in + T * D * ea
    if role == "x":
        return 0, T * D * ea + T * D
    return 0, 0


def backward_work(role, cfg, touched):
    """(flops, bytes) of one launch of a backward-pass span (bf16 plain layer): each GEMM's
    reduction over the real pairs only (per-expert padding adds zeros, not counted), touched
    expert weights read once, activations in and out once."""
    T, H, E, k, I, Is, L = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.latent
    P = T * k
    D = L or H                        # the experts' width
    wt = touched * I * D * 2          # one touched projection stack, bf16
    H0 = H
    H = D                             # routed products below run in the experts' width
    gemm = {
        # forward recompute: relu(a) and h saved, expert outputs Y
        "bwd_routed_up": (2 * P * I * H, wt + T * H * 2 + 2 * P * I * 2),
        "bwd_routed_down": (2 * P * H * I, wt + P * I * 2 + P * H * 2),
        "bwd_shared_up": (2 * T * Is * H0, Is * H0 * 2 + T * H0 * 2 + 2 * T * Is * 2),
        # data gradients (weights read as stored; the squared ReLU's derivative fused)
        "bwd_routed_dgrad_down": (2 * P * I * H, wt + P * H * 2 + 2 * P * I * 2),
        "bwd_routed_dgrad_up": (2 * P * H * I, wt + P * I * 2 + P * H * 4),
        "bwd_shared_dgrad_down": (2 * T * Is * H0, Is * H0 * 2 + T * H0 * 2 + 2 * T * Is * 2),
        "bwd_shared_dgrad_up": (2 * T * H0 * Is, H0 * Is * 2 + T * Is * 2 + T * H0 * 4),
        # weight gradients over each expert's pairs (fp32 out, every expert's matrix written)
        "bwd_routed_wgrad_down": (2 * P * H * I, P * H * 2 + P * I * 2 + E * H * I * 4),
        "bwd_routed_wgrad_up": (2 * P * I * H, P * I * 2 + P * H * 2 + E * I * H * 4),
        "bwd_shared_wgrad_down": (2 * T * H0 * Is, T * H0 * 2 + T * Is * 2 + H0 * Is * 4),
        "bwd_shared_wgrad_up": (2 * T * Is * H0, T * Is * 2 + T * H0 * 2 + Is * H0 * 4),
        # LatentMoE projections: dz = dy W_out, dW_out = dy^T z, dx += du W_in, dW_in = du^T x
        "bwd_latent_out_dgrad": (2 * T * L * H0, T * H0 * 2 + H0 * L * 2 + T * L * 2),
        "bwd_latent_out_wgrad": (2 * H0 * L * T, T * H0 * 2 + T * L * 2 + H0 * L * 4),
        "bwd_latent_in_dgrad": (2 * T * H0 * L, T * L * 2 + L * H0 * 2 + T * H0 * 4),
        "bwd_latent_in_wgrad": (2 * L * H0 * T, T * L * 2 + T * H0 * 2 + L * H0 * 4),
    }
    if role in gemm:
        f, b = gemm[role]
        return f, int(b)
    if role == "pairs":               # expert inputs gathered into pair order
        return 0, 2 * P * D * 2
    if role == "gates":               # dy, Y rows in; g*dy rows and dz out
        return 2 * P * D, T * D * 2 + P * D * 2 + P * D * 2 + P * 4
    if role == "du":                  # pair rows summed per token (LatentMoE)
        return P * D, P * D * 4 + T * D * 2
    if role == "dx":
        return P * H0 * 4, (T * H0 * 4 if Is else 0) + (T * H0 * 4 if L else P * H0 * 4) + \
            P * H0 * 2 + T * H0 * 4
    if role == "dW_r":
        return 2 * P * H0, P * 4 + P * H0 * 2 + E * H0 * 4
    return 0, 0


def backward_flops(cfg):
    """Algorithmic flops of the backward pass proper: data and weight gradients of the routed and
    shared experts, of the LatentMoE projections and of the router (the forward recompute is not
    counted)."""
    T, H, E, k, I, Is, L = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.latent
    P, D = T * k, cfg.D
    return 4 * 2 * P * I * D + 4 * 2 * T * Is * H + 4 * 2 * T * L * H + 2 * 2 * P * H + 2 * P * D


def kernel_of(span):
    return span.split(":")[0]


def mfma_dtype(kernel, cfg):
    # the block-scaled kernels multiply MXFP4 / MXFP8 weights by e4m3 tokens: fp8 rate
    if "fp8" in kernel or "e4m3" in kernel or "mxfp" in kernel:
        return "fp8"
    return "f32" if cfg.act_dtype == "f32" else "bf16"


# ------------------------------------------------------------------ one workload

def weights_key(cfg):
    """Workloads with equal keys draw the same seeded weights (only x and the bias differ)."""
    return (cfg.H, cfg.E, cfg.I, cfg.I_shared, cfg.latent, cfg.act_dtype, cfg.expert_dtype)


def prepare(name, moe, mi, torch, path, cache=None, wgrad_bf16=True):
    backward = name.endswith("+backward")
    cfg = mi.CONFIGS[name.split("+")[0]]
    key = weights_key(cfg)
    if cache is not None and key in cache:
        inp0, dev0 = cache[key]
        inp = mi.make_layer(cfg, 0, tensors={"x", "b"})       # same seeded weights: reuse them
        dev = dict(dev0)
        dev.update(moe.to_device(inp))
        inp = dict(inp0, **{k_: v for k_, v in inp.items()})
    else:
        inp = mi.make_layer(cfg, 0)
        dev = moe.to_device(inp)
        if cache is not None:
            cache[key] = (inp, dev)
    rt = moe.alloc_routing(cfg.T, cfg.E, cfg.k, "cuda")
    if backward:
        # the backward pass of the layer for a seeded upstream gradient dy, as a training step
        # runs it: after moe_layer_forward_train, reading the activations that call saved. The
        # forward call below records the routing (the same selection) for the byte counts.
        moe.layer_from(dev, cfg.k, path="grouped", routing=rt)()
        dy = moe.to_device({"dy": mi.make_grad_output(cfg, 0)})["dy"]
        bw = moe.backward_from(dev, cfg.k)
        bw.forward_train()
        w = dict(cfg=cfg, inp=inp, dev=dev, rt=rt, layer=lambda: bw(dy, saved=True),
                 recompute=lambda: bw(dy), train_forward=bw.forward_train, backward=True,
                 name=name)
        if wgrad_bf16:
            # the same pass writing the expert weight gradients in bf16 (MOE_WGRAD_BF16)
            bw16 = moe.backward_from(dev, cfg.k, wgrad_bf16=True)
            bw16.forward_train()
            w["wgrad_bf16"] = lambda: bw16(dy, saved=True)
        return w
    layer = moe.layer_from(dev, cfg.k, path=path, routing=rt)
    return dict(cfg=cfg, inp=inp, dev=dev, rt=rt, layer=layer, name=name)


def measure(w, moe, torch, steps, warmup, graph):
    cfg, layer = w["cfg"], w["layer"]
    stream = torch.cuda.current_stream()
    for _ in range(max(warmup, 1)):
        layer()
    torch.cuda.synchronize()
    counts = w["rt"]["counts"].cpu().numpy()

    # traced pass over a few steps: per-span durations, to find the dominant kernel
    spans_per_step = 32 if w.get("backward") else 16
    moe.binding.trace_enable(4 * spans_per_step)
    for _ in range(3):
        layer()
    torch.cuda.synchronize()
    recs = moe.binding.trace_records()
    moe.binding.trace_disable()
    per_kernel = {}
    for n, ms in recs:
        per_kernel.setdefault(kernel_of(n), 0.0)
        per_kernel[kernel_of(n)] += ms
    dominant = max(per_kernel, key=per_kernel.get)
    dispatch_launch = None
    runner = layer
    if graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            layer()                                 # warm the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            layer()
        torch.cuda.synchronize()
        runner = g.replay
        for _ in range(max(warmup, 1)):
            runner()
        torch.cuda.synchronize()

    # timed region: K steps; events bracket the dominant kernel's launches (eager mode)
    if not graph:
        moe.binding.trace_enable(steps * 8, dominant + ":")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        runner()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if not graph:
        krec = moe.binding.trace_records()
        moe.binding.trace_disable()
    else:
        # graph replays cannot carry the event records: time the kernel in an eager pass
        moe.binding.trace_enable(steps * 8, dominant + ":")
        for _ in range(steps):
            layer()
        torch.cuda.synchronize()
        krec = moe.binding.trace_records()
        moe.binding.trace_disable()
    ms_step = elapsed * 1e3 / steps
    stream_path = any(kernel_of(n) == "stream" for n, _ in recs)
    flops = sum(work_of(n, cfg, counts, stream_path)[0] for n, _ in krec)
    bts = sum(work_of(n, cfg, counts, stream_path)[1] for n, _ in krec)
    kms = sum(ms for _, ms in krec)
    nlaunch = len(krec)
    dt = mfma_dtype(dominant, cfg)
    ridge = PEAK_MFMA[dt] / PEAK_HBM
    ai = flops / max(bts, 1)
    if ai < ridge:
        bound, achieved, peak, unit = "hbm", bts / (kms * 1e-3) / 1e9, PEAK_HBM / 1e9, "GB/s"
    else:
        bound, achieved = "mfma", flops / (kms * 1e-3) / 1e12
        peak, unit = PEAK_MFMA[dt] / 1e12, "TFLOP/s"
    traffic = measured_traffic(w.get("name", cfg.name), dominant)
    roof = dict(bound=bound, achieved=round(achieved, 1), peak=peak, unit=unit,
                frac=round(achieved / peak, 4), traffic=traffic, kernel=dominant,
                launches=nlaunch, avg_launch_us=round(kms * 1e3 / max(nlaunch, 1), 2),
                algorithmic_flops_per_launch=int(flops / max(nlaunch, 1)),
                algorithmic_bytes_per_launch=int(bts / max(nlaunch, 1)))
    if traffic:
        roof["traffic_over_algorithmic_bytes"] = round(traffic / max(bts / max(nlaunch, 1), 1), 3)
    breakdown = {k_: round(v * 1e3 / 3, 2) for k_, v in sorted(per_kernel.items(),
                                                              key=lambda kv: -kv[1])}
    # outside the timed region: the distribution of single steps (events on the call's stream,
    # which also waits for the side stream), and steps after the 256 MB Infinity Cache has been
    # overwritten by a 512 MB store, so that no weights stay cached between steps
    dist = step_times(layer, torch, max(steps, 20))
    # eviction by a read-only sweep of 512 MB (written once here, outside the timed steps), so
    # that no dirty flush lines are written back inside the step that follows
    flush = torch.zeros(128 << 20, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    cold = step_times(layer, torch, min(max(steps, 10), 30),
                      before=lambda: torch.sum(flush, dim=0, out=sink))
    del flush, sink
    pct = lambda a, q: round(float(np.percentile(a, q)), 1)
    extra = {}
    if w.get("backward"):   # the whole pass against the bf16 peak (recompute not counted)
        roof["pass_flops"] = backward_flops(cfg)
        roof["pass_frac_of_bf16_peak"] = round(
            backward_flops(cfg) / (ms_step * 1e-3) / PEAK_MFMA["bf16"], 4)
        # the same backward recomputing the routing and expert activations itself, and the
        # training forward that saves them (median single steps)
        rec = step_times(w["recompute"], torch, max(steps // 2, 10))
        fwd = step_times(w["train_forward"], torch, max(steps // 2, 10))
        extra = dict(backward_recompute_us=round(float(np.median(rec)), 1),
                     forward_train_us=round(float(np.median(fwd)), 1))
        if "wgrad_bf16" in w:
            wg16 = float(np.median(step_times(w["wgrad_bf16"], torch, max(steps, 20))))
            extra.update(backward_wgrad_bf16_us=round(wg16, 1),
                         backward_wgrad_bf16_frac_of_bf16_peak=round(
                             backward_flops(cfg) / (wg16 * 1e-6) / PEAK_MFMA["bf16"], 4))
    step = None
    if not w.get("backward"):
        step = step_roofline(cfg, counts, float(np.median(dist)), float(np.median(cold)))
    return dict(ms_per_step=ms_step, tokens_per_s=cfg.T / (ms_step * 1e-3), roofline=roof,
                kernel_us_per_step=breakdown, touched_experts=int(np.count_nonzero(counts)),
                step_roofline=step,
                step_us=dict(median=pct(dist, 50), p10=pct(dist, 10), p90=pct(dist, 90),
                             cold_cache_median=pct(cold, 50),
                             cold_cache_tokens_per_s=round(cfg.T / (np.median(cold) * 1e-6), 1),
                             **extra))


def step_work(cfg, counts):
    """(flops by matrix-core dtype, bytes) of one whole layer call: the router over all E, the
    selected pairs' expert products, the shared expert and the latent projections; each touched
    expert's weights, the shared expert, router and projections read once, x read and y written
    once. 8- and 4-bit experts multiply e4m3 token rows (fp8 rate); the rest runs in the
    activation dtype."""
    T, H, E, k, I, Is, L, D = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.latent, cfg.D
    P = T * k
    ea = 4 if cfg.act_dtype == "f32" else 2
    ew = {"f32": 4, "bf16": 2, "e4m3": 1, "mxfp8": 1, "mxfp4": 0.5}[cfg.expert_dtype]
    narrow = cfg.expert_dtype in ("e4m3", "mxfp4", "mxfp8")
    touched = int(np.count_nonzero(counts))
    act = "f32" if cfg.act_dtype == "f32" else "bf16"
    flops = {act: 2 * T * E * H + 4 * T * Is * H + 4 * T * L * H}
    routed = 4 * P * I * D
    flops["fp8" if narrow else act] = flops.get("fp8" if narrow else act, 0) + routed
    scale = 0
    if cfg.expert_dtype == "e4m3":
        scale = touched * (I + D) * 4
    elif cfg.expert_dtype in ("mxfp4", "mxfp8"):
        scale = touched * 2 * I * D // 32
    b = touched * 2 * I * D * ew + scale + 2 * Is * H * ea + E * H * ea + 2 * L * H * ea + \
        2 * T * H * ea
    return flops, int(b)


def step_roofline(cfg, counts, warm_us, cold_us):
    """The whole step against its roofline: the larger of the HBM time of its algorithmic bytes
    and the matrix-core time of its flops (each dtype at its own dense peak); frac is that ideal
    time over the measured median step, warm and after the read-only eviction."""
    flops, b = step_work(cfg, counts)
    t_hbm = b / PEAK_HBM
    t_mfma = sum(f / PEAK_MFMA[dt] for dt, f in flops.items())
    ideal = max(t_hbm, t_mfma)
    return dict(bound="hbm" if t_hbm >= t_mfma else "mfma",
                algorithmic_bytes=b, algorithmic_flops={dt: int(f) for dt, f in flops.items()},
                ideal_us=round(ideal * 1e6, 1), frac=round(ideal / (warm_us * 1e-6), 4),
                frac_cold=round(ideal / (cold_us * 1e-6), 4))


def step_times(layer, torch, n, before=None):
    """Microseconds of n single steps, each bracketed by events on the current stream."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for a, b in ev:
        if before is not None:
            before()
        a.record()
        layer()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) * 1e3 for a, b in ev])


def peak_from_clock():
    """Dense peaks recomputed from the device's reported peak clock and CU count (4096 bf16 and
    8192 fp8 flops per CU per clock on gfx950), beside the published figures."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return None
    clk, cus = ctypes.c_int(0), ctypes.c_int(0)
    if hip.hipDeviceGetAttribute(ctypes.byref(clk), 5, 0) or \
            hip.hipDeviceGetAttribute(ctypes.byref(cus), 63, 0):   # clock rate (kHz), CU count
        return None
    hz = clk.value * 1e3
    return dict(clock_mhz=round(hz / 1e6), cus=cus.value,
                bf16_tflops=round(cus.value * 4096 * hz / 1e12, 1),
                fp8_tflops=round(cus.value * 8192 * hz / 1e12, 1))


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (profiles/traffic.json, copy-calibrated), or None when there is no entry or
    the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        ent = json.load(f)["entries"].get(f"{workload}/{kernel}")
    if ent is None:
        return None
    h = hashlib.sha256()
    for src in ent["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest()[:16] != ent["sha"]:
        return None
    return int(ent["traffic_bytes_per_launch"])


def cpu_baseline(w, n_tokens):
    from oracle import oracle as O
    cfg, inp = w["cfg"], w["inp"]
    toks = np.linspace(0, cfg.T - 1, n_tokens).astype(np.int32)
    O.build()
    t0 = time.perf_counter()
    O.forward(inp, toks)      # exact weights, one thread
    dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return dict(value=round(n_tokens / dt, 3), unit="tokens/s", cores=1, kind="oracle",
                cpu_model=model, host_cpus=os.cpu_count(),
                sample=f"{n_tokens} of the {cfg.T} tokens of {cfg.name} (router over all E, "
                       f"k experts and the shared expert per token), double precision, one "
                       f"thread, {dt:.1f} s; tokens are independent, so the rate extrapolates "
                       f"linearly to the whole batch")


def dtype_of(cfg):
    """Arithmetic types of the path: bf16, or the expert-weight format with bf16 activations."""
    if cfg.expert_dtype in ("e4m3", "mxfp4", "mxfp8"):
        return f"{cfg.expert_dtype}+bf16"
    return cfg.act_dtype


def describe(cfg):
    return dict(workload=cfg.name, description=cfg.description, T=cfg.T, H=cfg.H, E=cfg.E,
                k=cfg.k, I=cfg.I, I_shared=cfg.I_shared, latent=cfg.latent,
                act_dtype=cfg.act_dtype, expert_dtype=cfg.expert_dtype)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import moe_inputs as mi
    import sparse_moe_layer_05_amd as moe

    torch.cuda.set_device(0)
    moe.lib()
    cache = {}
    main_w = prepare(args.config, moe, mi, torch, args.path, cache, not args.no_wgrad_bf16)
    res = measure(main_w, moe, torch, args.steps, args.warmup, args.graph)
    print(f"[bench] {args.config}: {res['ms_per_step']:.4f} ms per step", file=sys.stderr,
          flush=True)
    cfg = main_w["cfg"]
    out = {
        "metric": METRIC, "value": round(res["tokens_per_s"], 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_of(cfg),
        "data": "synthetic", "config": describe(cfg), "roofline": res["roofline"],
    }
    extra = {}
    for name in [n for n in args.also.split(",") if n and n != args.config]:
        w = prepare(name, moe, mi, torch, args.path, cache, not args.no_wgrad_bf16)
        r = measure(w, moe, torch, args.steps, args.warmup, args.graph)
        extra[name] = dict(tokens_per_s=round(r["tokens_per_s"], 1), dtype=dtype_of(w["cfg"]),
                           ms_per_step=round(r["ms_per_step"], 4), roofline=r["roofline"],
                           step_roofline=r["step_roofline"], step_us=r["step_us"],
                           kernel_us_per_step=r["kernel_us_per_step"])
        if not args.no_cpu_baseline and not w.get("backward"):
            n = args.cpu_tokens or max(2, min(w["cfg"].T,
                                              int(ALSO_CPU_S / per_token_seconds(w["cfg"]))))
            extra[name]["cpu_baseline"] = cpu_baseline(w, n)
        print(f"[bench] {name}: {r['ms_per_step']:.4f} ms per step", file=sys.stderr, flush=True)
        del w
        torch.cuda.empty_cache()
    out["step_roofline"] = res["step_roofline"]
    out["step_us"] = res["step_us"]
    out["peak_from_clock"] = peak_from_clock()
    out["kernel_us_per_step"] = res["kernel_us_per_step"]
    out["touched_experts"] = res["touched_experts"]
    if extra:
        out["also"] = extra
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        n = args.cpu_tokens or max(4, min(cfg.T, int(15.0 / per_token_seconds(cfg))))
        out["cpu_baseline"] = cpu_baseline(main_w, n)
    print(json.dumps(out), flush=True)


ALSO_CPU_S = 4.0    # oracle seconds per extra workload (the headline one gets ~15 s)


def per_token_seconds(cfg):
    """Rough oracle cost per token (for a CPU sample of at most ~15 s): ~2.5 ns per
    multiply-add on the GPU hosts' cores (measured: 37 Nano decode tokens in 7.2 s)."""
    D = cfg.D
    macs = cfg.E * cfg.H + cfg.k * 2 * cfg.I * D + 2 * cfg.I_shared * cfg.H
    if cfg.latent:
        macs += 2 * cfg.latent * cfg.H
    return macs * 2.5e-9


if __name__ == "__main__":
    main()
