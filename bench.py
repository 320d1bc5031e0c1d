#!/usr/bin/env python3
"""Throughput of the RWKV WKV operators on one MI355X.

One step = one rwkv6_wkv_fwd call (Finch, time-parallel mode) over the Finch
workload: B=8 sequences x T=4096 tokens x D=2560 channels (H=40 heads of 64),
bf16 r/k/v, fp32 per-token decay logits and fp32 state, inputs resident in
HBM.  The JSON line reports tokens*channels/s of the timed steps, the
roofline of the chunked kernel (algorithmic bytes / average kernel time vs
8 TB/s), the fp64 oracle timed on the host cores, and the other operators on
their own workloads under "paths" (RWKV-4 scan, Eagle chunked, and the
single-token decode steps of Finch, Eagle and RWKV-4).

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-paths]
                       [--skip-cpu] [--only PATH]
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

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix, vendor figure
FLUSH_BYTES = 1 << 30        # > 256 MiB Infinity Cache
CALIB_BYTES = 1 << 30        # streaming copy used to calibrate HBM counters

METRIC = "WKV tokens*channels/s & % HBM/MFMA roofline, Finch D2560 T4096; decode steps/s"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    # From idle, the GPU's power management first lowers the shader clock
    # under a sustained load (2400 MHz to about 2070 MHz) and then brings it
    # back over about a hundred prefill launches: the first launches after
    # an idle period run up to a fifth slower.  Before the warm-up steps each
    # path therefore runs back-to-back for this long; the headline also
    # reports the unsettled ("cold") figure it measured first.
    ap.add_argument("--settle-s", type=float, default=0.5)
    ap.add_argument("--skip-paths", action="store_true", help="time only the headline step")
    ap.add_argument("--skip-cpu", action="store_true", help="do not time the oracle")
    ap.add_argument("--only", choices=["finch", "eagle", "rwkv4", "serial", "decode", "decode_big",
                                       "eagle_decode",
                                       "rwkv4_decode", "finch_bwd", "finch_gated", "finch_lora",
                                       "finch_train", "calib", "stream"],
                    help="time one path only (for profiling)")
    ap.add_argument("--decode-steps", type=int, default=1024)
    return ap.parse_args()


def source_hash(name):
    """First 16 hex digits of the sha256 over a kernel source and the headers
    of this package that it includes, directly or through other headers, so
    that counters taken before a change to any of them no longer match."""
    import re
    csrc = os.path.join(ROOT, "linear_attention_rnn_wkv_amd", "csrc")
    h = hashlib.sha256()
    seen, todo = set(), [name]
    while todo:
        n = todo.pop(0)
        path = os.path.join(csrc, n)
        if n in seen or not os.path.isfile(path):
            continue
        seen.add(n)
        with open(path, "rb") as f:
            data = f.read()
        h.update(n.encode() + b"\0" + data)
        todo += [m.decode() for m in re.findall(rb'#include "([^"]+)"', data)]
    return h.hexdigest()[:16]


def measured_traffic(kernel_src, per_launch_key):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current source of the kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[per_launch_key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_hash(kernel_src):
        return None
    return rec.get("bytes_per_launch")


class Timer:
    """HIP events around each launch on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __enter__(self):
        s = self.torch.cuda.Event(enable_timing=True)
        s.record()
        self.pairs.append([s, None])
        return self

    def __exit__(self, *exc):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[-1][1] = e

    def ms(self):
        return [s.elapsed_time(e) for s, e in self.pairs]


def flush(torch, buf):
    # Read, not write, a buffer larger than the last-level caches: the inputs
    # are evicted without leaving dirty lines whose write-back would land in
    # the timed launch.
    buf.sum()


def settle(torch, launch, seconds):
    """Back-to-back launches for about `seconds` (the GPU's clocks settle)."""
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        launch()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return {"launches": n, "seconds": time.perf_counter() - t0}


def time_launches(torch, launch, steps, warmup, flush_buf=None, settle_s=0.0, cold=False):
    """Per-launch HIP-event times of `steps` launches after `warmup` untimed
    ones.  cold: first, from an idle GPU, the same warmup + steps without
    settling (reported under "cold"); settle_s: back-to-back launches before
    the warm-up."""
    out = {}
    if cold:
        timer = Timer(torch)
        for i in range(warmup + steps):
            if flush_buf is not None:
                flush(torch, flush_buf)
            if i < warmup:
                launch()
            else:
                with timer:
                    launch()
        torch.cuda.synchronize()
        ms = timer.ms()
        out["cold"] = {"kernel_ms_mean": sum(ms) / len(ms), "kernel_ms_min": min(ms),
                       "kernel_ms_max": max(ms), "per_launch_us": [round(m * 1e3, 1) for m in ms]}
    if settle_s > 0:
        out["settle"] = settle(torch, launch, settle_s)
    for _ in range(warmup):
        if flush_buf is not None:
            flush(torch, flush_buf)
        launch()
    torch.cuda.synchronize()
    timer = Timer(torch)
    t0 = time.perf_counter()
    for _ in range(steps):
        if flush_buf is not None:
            flush(torch, flush_buf)
        with timer:
            launch()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = timer.ms()
    out.update({"kernel_ms_mean": sum(ms) / len(ms), "kernel_ms_min": min(ms),
                "kernel_ms_max": max(ms), "wall_s": wall})
    return out


def time_rotating(torch, launches, steps, warmup, settle_s=0.0):
    """Mean time per launch of `steps` back-to-back launches that cycle
    through `launches` (each on its own copy of the inputs, so that a copy's
    bytes leave the last-level cache before it is used again), between two
    HIP events: per-launch events would add their own overhead to a launch
    of a few microseconds."""
    n = len(launches)
    i = 0

    def one():
        nonlocal i
        launches[i % n]()
        i += 1
    out = {}
    if settle_s > 0:
        out["settle"] = settle(torch, one, settle_s)
    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        one()
    e1.record()
    torch.cuda.synchronize()
    out.update({"kernel_ms_mean": e0.elapsed_time(e1) / steps,
                "wall_s": time.perf_counter() - t0, "copies": n})
    return out


# ---------------------------------------------------------------------------
# paths

def finch_bytes(B, T, H, N=64):
    tok = B * T * H * N
    return tok * (2 * 3 + 4 + 2) + 2 * B * H * N * N * 4 + H * N * 4


def eagle_bytes(B, T, H, N=64):
    tok = B * T * H * N
    return tok * (2 * 3 + 2) + 2 * B * H * N * N * 4 + 2 * H * N * 4


def rwkv4_bytes(B, T, C):
    return B * T * C * 12 + 2 * B * 3 * C * 4 + 2 * C * 4


def decode_bytes_per_step(B, H, N=64):
    tok = B * H * N
    return 2 * B * H * N * N * 4 + tok * (2 * 3 + 4 + 2) + H * N * 4


def eagle_decode_bytes_per_step(B, H, N=64):
    tok = B * H * N
    return 2 * B * H * N * N * 4 + tok * (2 * 3 + 2) + 2 * H * N * 4


def rwkv4_decode_bytes_per_step(B, C):
    return B * C * 12 + 2 * B * 3 * C * 4 + 2 * C * 4


def finch_bwd_bytes(B, T, H, N=64):
    # read r, k, v, d_o (bf16) and x (fp32); write d_r, d_k, d_v (bf16) and d_x
    # (fp32); the states in and out and their gradients; u and d_u
    tok = B * T * H * N
    return tok * (2 * 4 + 4 + 2 * 3 + 4) + 4 * B * H * N * N * 4 + 2 * H * N * 4


def finch_gated_bytes(B, T, H, N=64):
    # the forward's bytes, the gate (bf16) read, the norm weight and bias read
    return finch_bytes(B, T, H, N) + B * T * H * N * 2 + 2 * H * N * 4


def finch_lora_bytes(B, T, H, N=64):
    # the fused forward: the producer reads the block input (bf16) and
    # writes act(z A_omega) (64 bf16 per token); the chunked kernel reads r,
    # k, v and that factor and writes o; the states in and out; the
    # producer's weights and vectors once
    D, rows = H * N, B * T
    return (rows * D * 2 + 2 * rows * 64 * 2 + rows * D * (2 * 3 + 2)
            + 2 * B * H * N * N * 4 + (2 * D * 32 + 2 * D * 64) * 2 + 4 * D * 4 + H * N * 4)


def lora_producer_bytes(B, T, H, N=64):
    # the decay producer alone: the block input and the shift rows read, the
    # weights and vectors once, act(z A_omega) written (64 bf16 per token)
    D, rows = H * N, B * T
    return rows * D * 2 + B * D * 2 + (2 * D * 32 + D * 64) * 2 + 2 * D * 4 + rows * 64 * 2


def lora_wkv_bytes(B, T, H, N=64):
    # the chunked kernel fed by it: r, k, v read and o written (bf16), the
    # rank-64 factor once per token, B_omega, omega and u, the states
    D, rows = H * N, B * T
    return (rows * D * (2 * 3 + 2) + rows * 64 * 2 + 64 * D * 2 + D * 4 + H * N * 4
            + 2 * B * H * N * N * 4)


def finch_recompute_bytes(B, T, H, N=64, L=64):
    # the backward's state recomputation: read k, v (bf16), x (fp32) and the
    # initial states (the states need no r); write the state entering every
    # chunk and the last
    tok, nch = B * T * H * N, (T + L - 1) // L
    return tok * (2 * 2 + 4) + B * H * N * N * 4 + B * H * (nch + 1) * N * N * 4


def finch_reverse_bytes(B, T, H, N=64, L=64):
    # the reverse sweep: read r, k, v, d_o (bf16), x (fp32), u, the chunk
    # states and the final state's gradient; write d_r, d_k, d_v (bf16), d_x
    # (fp32), the initial state's gradient and the per-sequence d_u partials
    tok, nch = B * T * H * N, (T + L - 1) // L
    return (tok * (2 * 4 + 4 + 2 * 3 + 4) + B * H * (nch + 1) * N * N * 4
            + 2 * B * H * N * N * 4 + H * N * 4 + B * H * N * 4)


def chunk_mfma_flops(B, T, H, N=64, L=64):
    # per chunk and head, as executed: A^T (lower-triangular 16x16 tiles,
    # K = N), A V (causal K-blocks), Q S, Kh_hi V + Kh_lo V, all bf16 MFMA
    chunks = (T + L - 1) // L
    per_chunk = 2 * 16 * 16 * 32 * (2 * 10 + 4 * (1 + 1 + 2 + 2) + 8 * 4 + 16 * 4)
    return B * H * chunks * per_chunk


def run_finch(torch, W, S, H2D, args, cfg=4):
    spec = S.WORKLOADS[cfg]
    d = S.workload(cfg)
    g = H2D(d)
    o = torch.empty_like(g["r"])
    so = torch.empty_like(g["s0"])
    fn = W.rwkv6_wkv_fwd if cfg == 4 else W.rwkv5_wkv_fwd
    B, T, H = spec["B"], spec["T"], spec["H"]
    ws = W.new_workspace(W.fwd_workspace_bytes(B, T, H))

    def launch():
        fn(g["r"], g["k"], g["v"], g["x"], g["u"], state_in=g["s0"], state_out=so, o=o,
           workspace=ws)

    res = time_launches(torch, launch, args.steps, args.warmup, settle_s=args.settle_s,
                        cold=cfg == 4)
    W.workspace_status(ws)
    nbytes = finch_bytes(B, T, H) if cfg == 4 else eagle_bytes(B, T, H)
    sec = res["kernel_ms_mean"] / 1e3
    res.update({
        "workload": S.WORKLOAD_NAMES[cfg],
        "tokens_channels_per_s": B * T * H * 64 / sec,
        "algorithmic_bytes": nbytes,
        "hbm_GBps": nbytes / sec / 1e9,
        "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS,
        "mfma_TFLOPs": chunk_mfma_flops(B, T, H) / sec / 1e12,
        "mfma_frac": chunk_mfma_flops(B, T, H) / sec / 1e12 / MFMA_BF16_PEAK_TFS,
    })
    return res, d


def run_finch_gated(torch, W, S, H2D, args, d4=None):
    """The Finch forward with the output epilogue (LayerNorm per head, SiLU
    gate) fused into the output write."""
    spec = S.WORKLOADS[4]
    B, T, H = spec["B"], spec["T"], spec["H"]
    d = dict(d4) if d4 is not None else S.workload(4)
    d.update(S.epilogue_inputs(B, T, H, 64, 4))
    g = H2D(d)
    y = torch.empty_like(g["r"])
    so = torch.empty_like(g["s0"])
    ws = W.new_workspace(W.fwd_workspace_bytes(B, T, H))

    def launch():
        W.rwkv6_wkv_fwd_gated(g["r"], g["k"], g["v"], g["x"], g["u"], g["g"], g["ln_w"],
                              g["ln_b"], 1e-5, state_in=g["s0"], state_out=so, y=y,
                              workspace=ws)

    res = time_launches(torch, launch, args.steps, args.warmup, settle_s=args.settle_s)
    W.workspace_status(ws)
    nbytes = finch_gated_bytes(B, T, H)
    sec = res["kernel_ms_mean"] / 1e3
    res.update({"workload": "finch_fwd_gated_B8_T4096_D2560_H40_N64_bf16",
                "tokens_channels_per_s": B * T * H * 64 / sec,
                "algorithmic_bytes": nbytes, "hbm_GBps": nbytes / sec / 1e9,
                "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS})
    return res


def run_finch_lora(torch, W, S, H2D, args, d4=None):
    """Finch workload with the decay logits made on the device from a block
    input by ddlerp and LoRA_omega (tanh): the producer and the chunked
    kernel, timed together as one call."""
    spec = S.WORKLOADS[4]
    B, T, H = spec["B"], spec["T"], spec["H"]
    d = dict(d4) if d4 is not None else S.workload(4)
    d.update(S.decay_lora_inputs(B, T, H, 64, 4))
    g = H2D({n: a for n, a in d.items() if a is not None})
    o = torch.empty_like(g["r"])
    so = torch.empty_like(g["s0"])
    ws = W.new_workspace(W.fwd_lora_workspace_bytes(B, T, H))

    def launch():
        W.rwkv6_wkv_fwd_lora(g["r"], g["k"], g["v"], g["xin"], g["mu_x"], g["lam"], g["A1"],
                             g["B1"], g["omega"], g["A2"], g["B2"], g["u"], act="tanh",
                             shift=g["shift"], state_in=g["s0"], state_out=so, o=o,
                             workspace=ws)

    res = time_launches(torch, launch, args.steps, args.warmup, settle_s=args.settle_s)
    W.workspace_status(ws)
    nbytes = finch_lora_bytes(B, T, H)
    sec = res["kernel_ms_mean"] / 1e3
    res.update({"workload": "finch_fwd_lora_B8_T4096_D2560_H40_N64_bf16",
                "tokens_channels_per_s": B * T * H * 64 / sec,
                "algorithmic_bytes": nbytes, "hbm_GBps": nbytes / sec / 1e9,
                "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS})

    # The same result in two calls: the producer writes the fp32 logits, the
    # plain chunked forward reads them
    dl = torch.empty((B, T, H * 64), dtype=torch.float32, device="cuda")
    lws = torch.empty(W.lora_workspace_bytes(B, T, H * 64), dtype=torch.uint8, device="cuda")
    fws = W.new_workspace(W.fwd_workspace_bytes(B, T, H))

    def two_calls():
        W.rwkv6_decay_lora(g["xin"], g["mu_x"], g["lam"], g["A1"], g["B1"], g["omega"],
                           g["A2"], g["B2"], act="tanh", shift=g["shift"], d=dl, workspace=lws)
        W.rwkv6_wkv_fwd(g["r"], g["k"], g["v"], dl.view(B, T, H, 64), g["u"],
                        state_in=g["s0"], state_out=so, o=o, workspace=fws)

    two = time_launches(torch, two_calls, args.steps, args.warmup, settle_s=args.settle_s)
    W.workspace_status(fws)
    res["two_calls"] = {"kernel_ms_mean": two["kernel_ms_mean"],
                        "kernel_ms_min": two["kernel_ms_min"],
                        "note": "rwkv6_decay_lora (fp32 logits to memory) + rwkv6_wkv_fwd",
                        "fused_speedup": two["kernel_ms_mean"] / res["kernel_ms_mean"]}
    return res


def run_finch_train(torch, W, S, H2D, args, d4=None):
    """One training step of the operator on the Finch workload: the forward
    that keeps the chunk states, then the backward that reads them (the
    states are not recomputed), timed together."""
    spec = S.WORKLOADS[4]
    B, T, H = spec["B"], spec["T"], spec["H"]
    d = dict(d4) if d4 is not None else S.workload(4)
    d.update(S.grad_inputs(B, T, H, 64, 4))
    g = H2D(d)
    ws = W.new_workspace(W.workspace_bytes(B, T, H))
    o = torch.empty_like(g["r"])
    so = torch.empty_like(g["s0"])
    grads = {"d_r": torch.empty_like(g["r"]), "d_k": torch.empty_like(g["r"]),
             "d_v": torch.empty_like(g["r"]), "d_x": torch.empty_like(g["x"]),
             "d_u": torch.empty_like(g["u"]), "d_state_in": torch.empty_like(g["s0"])}

    def launch():
        W.rwkv6_wkv_fwd_save(g["r"], g["k"], g["v"], g["x"], g["u"], ws, state_in=g["s0"],
                             state_out=so, o=o)
        W.rwkv6_wkv_bwd_saved(g["r"], g["k"], g["v"], g["x"], g["u"], g["d_o"], ws,
                              d_state_out=g["d_sT"], grads=grads)

    res = time_launches(torch, launch, max(10, args.steps // 2), max(5, args.warmup // 2),
                        settle_s=args.settle_s)
    W.workspace_status(ws)
    nch = (T + 63) // 64
    nbytes = finch_bytes(B, T, H) + B * H * (nch + 1) * 64 * 64 * 4 + finch_reverse_bytes(B, T, H)
    sec = res["kernel_ms_mean"] / 1e3
    res.update({"workload": "finch_train_step_B8_T4096_D2560_H40_N64_bf16",
                "tokens_channels_per_s": B * T * H * 64 / sec,
                "algorithmic_bytes": nbytes, "hbm_GBps": nbytes / sec / 1e9,
                "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS})
    return res


def run_finch_bwd(torch, W, S, H2D, args, d4=None):
    """Backward of the Finch workload: the state recomputation (a forward
    pass that stores the state entering every chunk), the reverse sweep and
    the sums over sequences, timed together as one call."""
    spec = S.WORKLOADS[4]
    B, T, H = spec["B"], spec["T"], spec["H"]
    d = dict(d4) if d4 is not None else S.workload(4)
    d.update(S.grad_inputs(B, T, H, 64, 4))
    g = H2D(d)
    ws = W.new_workspace(W.workspace_bytes(B, T, H))
    grads = {"d_r": torch.empty_like(g["r"]), "d_k": torch.empty_like(g["r"]),
             "d_v": torch.empty_like(g["r"]), "d_x": torch.empty_like(g["x"]),
             "d_u": torch.empty_like(g["u"]), "d_state_in": torch.empty_like(g["s0"])}

    def launch():
        W.rwkv6_wkv_bwd(g["r"], g["k"], g["v"], g["x"], g["u"], g["d_o"], state_in=g["s0"],
                        d_state_out=g["d_sT"], grads=grads, workspace=ws)

    res = time_launches(torch, launch, max(10, args.steps // 2), max(5, args.warmup // 2),
                        settle_s=args.settle_s)
    W.workspace_status(ws)
    nbytes = finch_bwd_bytes(B, T, H)
    sec = res["kernel_ms_mean"] / 1e3
    res.update({"workload": "finch_bwd_B8_T4096_D2560_H40_N64_bf16",
                "tokens_channels_per_s": B * T * H * 64 / sec,
                "algorithmic_bytes": nbytes, "hbm_GBps": nbytes / sec / 1e9,
                "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS,
                "workspace_bytes": ws.numel(),
                "note": "one call = state recomputation + reverse sweep + sums"})
    return res


# 32 x 75.65 MB = 2.4 GB between two uses of a copy.  With the kernel's
# non-temporal loads, 8 copies (605 MB) still let part of the inputs come from
# the 256 MB cache (18.4 against 19.4 us per launch); 32 and more read HBM.
RWKV4_COPIES = 32


def run_rwkv4(torch, W, S, H2D, args, flush_buf):
    """RWKV-4 scan, B8 T1024 C768.  Main figure: back-to-back launches that
    cycle through RWKV4_COPIES copies of the inputs and outputs (each launch
    reads its k, v from HBM), timed between two events.  Also: single launches after a
    read of a 1 GiB buffer that evicts the caches, each between its own pair
    of events (that figure includes the events' own overhead)."""
    spec = S.WORKLOADS[2]
    B, T, C = spec["B"], spec["T"], spec["C"]
    d = S.workload(2)
    k, v, w, u = (H2D({"a": d[n]})["a"] for n in ("k", "v", "w", "u"))
    nws = W.rwkv4_workspace_bytes(B, T, C)
    sets = []
    for i in range(RWKV4_COPIES):
        kc, vc = (k, v) if i == 0 else (k.clone(), v.clone())
        sets.append((kc, vc, torch.empty_like(k), torch.empty((B, 3, C), device="cuda"),
                     W.new_workspace(nws)))

    def launcher(kc, vc, y, so, ws):
        return lambda: W.rwkv4_wkv_fwd(kc, vc, w, u, state_out=so, y=y, workspace=ws)

    launches = [launcher(*st) for st in sets]
    res = time_rotating(torch, launches, max(args.steps, 20) * RWKV4_COPIES // 4, args.warmup,
                        settle_s=args.settle_s)
    iso = time_launches(torch, launches[0], max(args.steps, 20), min(args.warmup, 20), flush_buf)
    for st in sets:
        W.workspace_status(st[4])
    nbytes = rwkv4_bytes(B, T, C)
    sec = res["kernel_ms_mean"] / 1e3
    res.update({"workload": S.WORKLOAD_NAMES[2],
                "timing": f"back-to-back launches over {RWKV4_COPIES} copies of the "
                          "inputs and outputs, two events around them",
                "tokens_channels_per_s": B * T * C / sec,
                "algorithmic_bytes": nbytes, "hbm_GBps": nbytes / sec / 1e9,
                "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS,
                "isolated": {"cache": "flushed before each launch",
                             "kernel_ms_mean": iso["kernel_ms_mean"],
                             "kernel_ms_min": iso["kernel_ms_min"],
                             "hbm_frac": nbytes / (iso["kernel_ms_mean"] / 1e3) / 1e9
                                         / HBM_PEAK_GBS}})
    return res


def run_decode(torch, W, S, H2D, args, cfg=5, batch=None):
    """Back-to-back single-token steps: Finch (workload 5) over distinct
    per-step inputs; Eagle (6) and RWKV-4 (7) cycle through 64 distinct
    steps' inputs (the bytes each step moves are the same).  batch: Finch
    with that many sequences instead of 256, over 64 distinct steps."""
    spec = dict(S.WORKLOADS[cfg])
    if batch is not None:
        spec["B"] = batch
    steps = args.decode_steps
    distinct = steps if (cfg == 5 and batch is None) else min(steps, 64)
    d = S.workload(cfg, steps=distinct, B=spec["B"])
    g = H2D(d)
    if cfg == 7:
        st = torch.zeros((spec["B"], 3, spec["C"]), device="cuda")
        st[:, 2] = -1e38
        s0 = st.clone()
        y = torch.empty_like(g["k"])
        views = [(g["k"][s].unsqueeze(1), g["v"][s].unsqueeze(1), y[s].unsqueeze(1))
                 for s in range(distinct)]

        def one(s):
            k, v, ys = views[s % distinct]
            W.rwkv4_wkv_step(k, v, g["w"], g["u"], st, y=ys)
        nbytes = rwkv4_decode_bytes_per_step(spec["B"], spec["C"])
    else:
        st = g["s0"].clone()
        s0 = g["s0"]
        o = torch.empty_like(g["r"])
        per_token = cfg == 5
        views = [(g["r"][s].unsqueeze(1), g["k"][s].unsqueeze(1), g["v"][s].unsqueeze(1),
                  g["x"][s].unsqueeze(1) if per_token else g["x"], o[s].unsqueeze(1))
                 for s in range(distinct)]
        step = W.rwkv6_wkv_step if per_token else W.rwkv5_wkv_step

        def one(s):
            r, k, v, x, os_ = views[s % distinct]
            step(r, k, v, x, g["u"], st, o=os_)
        nbytes = (decode_bytes_per_step(spec["B"], spec["H"]) if per_token
                  else eagle_decode_bytes_per_step(spec["B"], spec["H"]))

    for s in range(min(8, steps)):  # warm-up on a scratch copy of the state
        one(s)
    settle(torch, lambda: one(0), args.settle_s)
    st.copy_(s0)
    torch.cuda.synchronize()
    timer = Timer(torch)
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(steps):
        with timer:
            one(s)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms = timer.ms()
    per = sum(ms) / len(ms)

    # The same steps replayed from a captured HIP graph: the interval then
    # measures the GPU rather than the Python launch rate, which bounds the
    # eager loop when a step takes only a few microseconds.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one(0)
    side.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for s in range(distinct):
            one(s)
    reps = max(1, steps // distinct)
    st.copy_(s0)
    graph.replay()
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(end) / (reps * distinct)
    name = S.WORKLOAD_NAMES[cfg]
    if batch is not None:
        name = name.replace(f"B{S.WORKLOADS[cfg]['B']}", f"B{batch}")
    return {"workload": name, "steps": reps * distinct,
            "distinct_steps": distinct, "timing": "graph replay",
            "steps_per_s": 1e3 / graph_ms, "ms_per_step": graph_ms,
            "algorithmic_bytes_per_step": nbytes,
            "hbm_GBps": nbytes / (graph_ms / 1e3) / 1e9,
            "hbm_frac": nbytes / (graph_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
            "eager": {"steps": steps, "steps_per_s": steps / (total_ms / 1e3),
                      "interval_ms": total_ms, "kernel_ms_mean": per, "wall_s": wall}}


def run_serial_segments(torch, W, S, H2D, args, T=64):
    """The serial (decode) kernel applying T tokens per call to 256 x 64 heads
    whose states stay in registers through the call: the cost of carrying
    the state token by token, the arithmetic a chunked forward would repeat
    to make its carried state bit-identical to the serial mode's."""
    B, H = 256, 64
    d = S.wkv_inputs(B, T, H, 64, 5, True, 0.1)
    g = H2D(d)
    st = g["s0"].clone()
    o = torch.empty_like(g["r"])

    def launch():
        W.rwkv6_wkv_step(g["r"], g["k"], g["v"], g["x"], g["u"], st, o=o)

    res = time_launches(torch, launch, max(10, args.steps // 4), args.warmup,
                        settle_s=args.settle_s)
    sec = res["kernel_ms_mean"] / 1e3
    token_heads = B * H * T
    res.update({"workload": f"finch_serial_B{B}_H{H}_T{T}",
                "ns_per_token_head": sec / token_heads * 1e9,
                "note": "each token: the output (4096 multiply-adds) and the state update "
                        "(4096 multiplies and 4096 fused multiply-adds) of one head"})
    return res


def cpu_baseline(S, d4, min_seconds=10.0):
    """The fp64 oracle on the whole Finch workload, all host threads, repeated
    until about `min_seconds` of CPU work have run (at least one pass)."""
    import oracle
    r, k, v = (S.bf16_to_f32(d4[n]) for n in ("r", "k", "v"))
    nthreads = oracle.default_threads()
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.wkv_matrix(r, k, v, d4["x"], d4["u"], d4["s0"], nthreads=nthreads)
        passes += 1
        sec = time.perf_counter() - t0
        if sec >= min_seconds:
            break
    B, T, H, N = d4["r"].shape
    # the RWKV-4 workloads, single-threaded
    single = {}
    for cfg in (1, 2):
        d = S.workload(cfg)
        reps = 0
        t1 = time.perf_counter()
        while True:
            oracle.rwkv4_fwd(d["k"], d["v"], d["w"], d["u"], nthreads=1)
            reps += 1
            el = time.perf_counter() - t1
            if el >= 1.0:
                break
        b, t, c = d["k"].shape
        single[S.WORKLOAD_NAMES[cfg]] = {"seconds_per_pass": el / reps,
                                         "tokens_channels_per_s": reps * b * t * c / el,
                                         "threads": 1}
    return {"value": passes * B * T * H * N / sec, "unit": "tokens*channels/s",
            "cores": nthreads, "kind": "oracle", "seconds": sec,
            "sample": f"the full Finch workload (B={B}, T={T}, H={H}, N={N}), "
                      f"{passes} passes",
            "cpu_model": cpu_model(), "single_thread": single}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ---------------------------------------------------------------------------
# counter summaries

PMC_PATHS = {  # bench path -> (kernel name fragment, source file, algorithmic bytes)
    "finch_fwd": ("wkv_chunk_kernel<true,", "wkv_chunk.hip", lambda: finch_bytes(8, 4096, 40)),
    "eagle_fwd": ("wkv_chunk_kernel<false,", "wkv_chunk.hip", lambda: eagle_bytes(8, 4096, 32)),
    "rwkv4_fwd": ("rwkv4_chain_kernel", "rwkv4_scan.hip", lambda: rwkv4_bytes(8, 1024, 768)),
    "finch_fwd_gated": ("wkv_chunk_kernel<true, 8, false, true, false>", "wkv_chunk.hip",
                        lambda: finch_gated_bytes(8, 4096, 40)),
    "finch_bwd_recompute": ("wkv_chunk_kernel<true, 8, true, false, false>", "wkv_chunk.hip",
                            lambda: finch_recompute_bytes(8, 4096, 40)),
    "finch_bwd_reverse": ("wkv_bwd_kernel<true>", "wkv_chunk_bwd.hip",
                          lambda: finch_reverse_bytes(8, 4096, 40)),
    "finch_lora_producer": ("decay_once_kernel<true, 5, false>", "decay_lora.hip",
                            lambda: lora_producer_bytes(8, 4096, 40)),
    "finch_lora_wkv": ("wkv_chunk_kernel<true, 8, false, false, true>", "wkv_chunk.hip",
                       lambda: lora_wkv_bytes(8, 4096, 40)),
    "finch_decode": ("wkv_step_kernel<true, false>", "wkv_step.hip",
                     lambda: decode_bytes_per_step(256, 64)),
    "eagle_decode": ("wkv_step_kernel<false, false>", "wkv_step.hip",
                     lambda: eagle_decode_bytes_per_step(256, 64)),
    "rwkv4_decode": ("rwkv4_decode4_kernel", "rwkv4_step.hip",
                     lambda: rwkv4_decode_bytes_per_step(256, 4096)),
    "finch_decode_B1024": ("wkv_step_kernel<true, true>", "wkv_step.hip",
                           lambda: decode_bytes_per_step(1024, 64)),
}
PMC_DIRS = {"finch_fwd": "finch", "eagle_fwd": "eagle", "rwkv4_fwd": "rwkv4",
            "finch_fwd_gated": "finch_gated", "finch_bwd_recompute": "finch_bwd",
            "finch_bwd_reverse": "finch_bwd", "finch_lora_producer": "finch_lora",
            "finch_lora_wkv": "finch_lora",
            "finch_decode": "decode", "eagle_decode": "eagle_decode",
            "rwkv4_decode": "rwkv4_decode", "finch_decode_B1024": "decode_big"}


def _pmc_mean(csv_path, fragment, counter):
    import csv
    vals = []
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if fragment in row["Kernel_Name"] and row["Counter_Name"] == counter:
                vals.append(float(row["Counter_Value"]))
    return sum(vals) / len(vals) if vals else None, len(vals)


def summarize_pmc(pmc_dir):
    """Turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (one directory per
    path and counter: <pmc_dir>/<path>_<COUNTER>/run_counter_collection.csv,
    made by `rocprofv3 --pmc <COUNTER> --output-format csv -d <that dir>
    -o run -- python bench.py --only <path> --steps 2 --warmup 1 --skip-cpu
    --decode-steps 8`) into profiles/traffic.json: HBM bytes per launch,
    scaled by the same counters on a 1 GiB streaming kernel (--only calib)."""
    csv_of = lambda tag, ctr: os.path.join(pmc_dir, f"{tag}_{ctr}", "run_counter_collection.csv")
    cal_f, _ = _pmc_mean(csv_of("calib", "FETCH_SIZE"), "MulFunctor", "FETCH_SIZE")
    cal_w, _ = _pmc_mean(csv_of("calib", "WRITE_SIZE"), "MulFunctor", "WRITE_SIZE")
    kib = CALIB_BYTES / 1024
    out = {"calibration": {
        "kernel": "torch.mul(a, 1.0, out=b) over 1 GiB fp32 (reads 1 GiB, writes 1 GiB)",
        "FETCH_SIZE_KiB": cal_f, "WRITE_SIZE_KiB": cal_w,
        "fetch_factor": kib / cal_f, "write_factor": kib / cal_w}}
    for path, (frag, src, alg) in PMC_PATHS.items():
        tag = PMC_DIRS[path]
        f, nf = _pmc_mean(csv_of(tag, "FETCH_SIZE"), frag, "FETCH_SIZE")
        w, nw = _pmc_mean(csv_of(tag, "WRITE_SIZE"), frag, "WRITE_SIZE")
        if f is None or w is None:
            continue
        rd = f * 1024 * out["calibration"]["fetch_factor"]
        wr = w * 1024 * out["calibration"]["write_factor"]
        out[path] = {"kernel": frag, "source": src, "source_sha256_16": source_hash(src),
                     "dispatches": [nf, nw], "FETCH_SIZE_KiB": f, "WRITE_SIZE_KiB": w,
                     "read_bytes": rd, "write_bytes": wr, "bytes_per_launch": rd + wr,
                     "algorithmic_bytes": alg(), "traffic_over_algorithmic": (rd + wr) / alg()}
    dst = os.path.join(ROOT, "profiles", "traffic.json")
    with open(dst, "w") as fh:
        json.dump(out, fh, indent=1)
    return out


def summarize_trace(csv_path):
    """Markdown table of a rocprofv3 --kernel-trace --stats kernel_stats.csv
    (durations in ns there, microseconds here), longest total first."""
    import csv
    rows = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]),
                         float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"])))
    rows.sort(key=lambda x: -x[2])
    out = ["| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for name, calls, _, avg, mn, mx in rows:
        out.append(f"| {name[:120]} | {calls} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | "
                   f"{mx / 1e3:.1f} |")
    return "\n".join(out)


def measure_stream(torch, nbytes=1 << 30, reps=10):
    """Achievable HBM bandwidth on this GPU: plain streaming kernels
    (libstream_probe.so: 16-byte loads / stores, eight in flight per thread)
    reading, copying and writing 1 GiB buffers (four times the last-level
    cache), best launch shape and cache policy (plain or non-temporal loads
    and stores) of a small sweep, median of `reps` launches."""
    import ctypes
    from linear_attention_rnn_wkv_amd import _build
    L = ctypes.CDLL(_build.PROBE_LIBRARY)
    L.stream_probe.restype = ctypes.c_int
    L.stream_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                               ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    sink = torch.empty(1 << 14, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {"kind": "plain streaming kernels of this repository over 1 GiB buffers "
                   "(read; copy = read + write; write), best of a launch-shape and "
                   "cache-policy sweep",
           "bytes": nbytes}
    # probe kinds per operation: (kind, cache policy)
    kinds = {"read": ((0, "plain"), (3, "non-temporal")),
             "copy": ((1, "plain"), (6, "non-temporal loads"), (4, "non-temporal")),
             "write": ((2, "plain"), (5, "non-temporal"))}
    for name, moved in (("read", nbytes), ("copy", 2 * nbytes), ("write", nbytes)):
        best = None
        for (kind, policy), (blocks, threads) in ((kp, bt) for kp in kinds[name] for bt in (
                (1024, 256), (2048, 256), (4096, 256), (2048, 512))):
            dst = sink if name == "read" else b

            def go():
                st = L.stream_probe(kind, a.data_ptr(), dst.data_ptr(), nbytes, blocks, threads,
                                    stream)
                if st != 0:
                    raise RuntimeError(f"stream_probe({kind}) returned {st}")
            for _ in range(3):
                go()
            torch.cuda.synchronize()
            ms = []
            for _ in range(reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                go()
                e1.record()
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
            ms.sort()
            gbs = moved / (ms[len(ms) // 2] / 1e3) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, blocks, threads, policy)
        out[f"{name}_GBps"] = best[0]
        out[f"{name}_frac_of_peak"] = best[0] / HBM_PEAK_GBS
        out[f"{name}_launch"] = [best[1], best[2]]
        out[f"{name}_policy"] = best[3]
    out["copy_GBps_torch"] = measure_torch_copy(torch, a, b, reps)
    del a, b
    return out


def measure_torch_copy(torch, a, b, reps):
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    ms.sort()
    return 2 * a.numel() * 4 / (ms[len(ms) // 2] / 1e3) / 1e9


def main():
    if len(sys.argv) == 3 and sys.argv[1] == "--summarize-pmc":
        print(json.dumps(summarize_pmc(sys.argv[2]), indent=1))
        return 0
    if len(sys.argv) == 3 and sys.argv[1] == "--summarize-trace":
        print(summarize_trace(sys.argv[2]))
        return 0
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the operator shards by sequence and head, with no exchange between "
              "GPUs)", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import linear_attention_rnn_wkv_amd as W
    import wkv_synth as S

    W.lib()
    torch.cuda.set_device(0)

    def H2D(d):
        out = {}
        for n, a in d.items():
            a = np.ascontiguousarray(a)
            t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
            t = t.cuda()
            out[n] = t.view(torch.bfloat16) if a.dtype == np.uint16 else t
        return out

    paths = {}
    only = args.only
    if only == "stream":
        print(json.dumps(measure_stream(torch)))
        return 0
    if only == "calib":
        # a plain streaming kernel of known size: reads 1 GiB, writes 1 GiB;
        # its FETCH_SIZE / WRITE_SIZE readings calibrate the HBM counters
        a = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"calib_bytes": CALIB_BYTES}))
        return 0
    d4 = None
    if only in (None, "finch"):
        print("finch forward ...", file=sys.stderr, flush=True)
        finch, d4 = run_finch(torch, W, S, H2D, args, cfg=4)
        paths["finch_fwd"] = finch
    flush_buf = None
    if not args.skip_paths and only in (None, "eagle"):
        print("eagle forward ...", file=sys.stderr, flush=True)
        paths["eagle_fwd"], _ = run_finch(torch, W, S, H2D, args, cfg=3)
    if not args.skip_paths and only in (None, "rwkv4"):
        print("rwkv4 forward ...", file=sys.stderr, flush=True)
        flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        paths["rwkv4_fwd"] = run_rwkv4(torch, W, S, H2D, args, flush_buf)
        del flush_buf
    if not args.skip_paths and only in (None, "finch_gated"):
        print("finch forward with the epilogue ...", file=sys.stderr, flush=True)
        paths["finch_fwd_gated"] = run_finch_gated(torch, W, S, H2D, args, d4)
    if not args.skip_paths and only in (None, "finch_lora"):
        print("finch forward with the decay producer ...", file=sys.stderr, flush=True)
        paths["finch_fwd_lora"] = run_finch_lora(torch, W, S, H2D, args, d4)
    if not args.skip_paths and only in (None, "finch_bwd"):
        print("finch backward ...", file=sys.stderr, flush=True)
        paths["finch_bwd"] = run_finch_bwd(torch, W, S, H2D, args, d4)
    if not args.skip_paths and only in (None, "finch_train"):
        print("finch training step (forward keeping the states + backward) ...",
              file=sys.stderr, flush=True)
        paths["finch_train"] = run_finch_train(torch, W, S, H2D, args, d4)
    if not args.skip_paths and only in (None, "serial"):
        print("finch serial mode, 64 tokens per call ...", file=sys.stderr, flush=True)
        paths["finch_serial_T64"] = run_serial_segments(torch, W, S, H2D, args)
    if not args.skip_paths and only in (None, "decode"):
        print("finch decode ...", file=sys.stderr, flush=True)
        paths["finch_decode"] = run_decode(torch, W, S, H2D, args)
    if not args.skip_paths and only in (None, "decode_big"):
        # a state of 1.07 GB, four times the 256 MB last-level cache: every
        # step's state bytes come from HBM
        print("finch decode, 1024 sequences ...", file=sys.stderr, flush=True)
        paths["finch_decode_B1024"] = run_decode(torch, W, S, H2D, args, batch=1024)
    if not args.skip_paths and only in (None, "eagle_decode"):
        print("eagle decode ...", file=sys.stderr, flush=True)
        paths["eagle_decode"] = run_decode(torch, W, S, H2D, args, cfg=6)
    if not args.skip_paths and only in (None, "rwkv4_decode"):
        print("rwkv4 decode ...", file=sys.stderr, flush=True)
        paths["rwkv4_decode"] = run_decode(torch, W, S, H2D, args, cfg=7)
    torch.cuda.synchronize()

    if "finch_fwd" not in paths:
        print(json.dumps({"paths": paths}))
        return 0

    for key, rec in paths.items():  # counter-measured HBM bytes, while current
        if key in PMC_PATHS:
            rec["traffic_bytes"] = measured_traffic(PMC_PATHS[key][1], key)
    if "finch_fwd_lora" in paths:  # the producer and the chunked kernel, each on its own
        paths["finch_fwd_lora"]["traffic_bytes"] = {
            k: measured_traffic(PMC_PATHS[k][1], k)
            for k in ("finch_lora_producer", "finch_lora_wkv")}
    if "finch_bwd" in paths:  # the backward's two main kernels, each on its own
        paths["finch_bwd"]["traffic_bytes"] = {
            k: measured_traffic(PMC_PATHS[k][1], k)
            for k in ("finch_bwd_recompute", "finch_bwd_reverse")}
    # the same bandwidths against what plain streaming kernels reach on this
    # GPU (each path against the copy: it reads and writes, as they do)
    achievable = measure_stream(torch)
    for rec in paths.values():
        if "hbm_GBps" in rec:
            rec["hbm_frac_of_copy"] = rec["hbm_GBps"] / achievable["copy_GBps"]
    finch = paths["finch_fwd"]
    spec = S.WORKLOADS[4]
    cold = None
    if "cold" in finch:  # the same steps from an idle GPU, before the clocks settle
        c = finch.pop("cold")
        nb = finch["algorithmic_bytes"]
        cold = {"steps": args.steps, "warmup": args.warmup,
                "kernel_ms_mean": c["kernel_ms_mean"], "kernel_ms_min": c["kernel_ms_min"],
                "kernel_ms_max": c["kernel_ms_max"],
                "frac": nb / (c["kernel_ms_mean"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                "per_launch_us": c["per_launch_us"][:64],
                "note": "timed launches before the settle phase; value and roofline are "
                        "measured after it"}
    ms = finch["wall_s"] / args.steps * 1e3
    cpu = None
    if not args.skip_cpu:
        print("oracle on the host ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(S, d4)
    traffic = measured_traffic("wkv_chunk.hip", "finch_fwd")
    line = {
        "metric": METRIC,
        "value": spec["B"] * spec["T"] * spec["H"] * spec["N"] / (ms / 1e3),
        "unit": "tokens*channels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": S.WORKLOAD_NAMES[4], "B": spec["B"], "T": spec["T"],
                   "H": spec["H"], "N": spec["N"], "D": spec["H"] * spec["N"],
                   "state": "fp32", "decay_logits": "fp32 per token"},
        "roofline": {"bound": "hbm", "achieved": finch["hbm_GBps"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": finch["hbm_frac"], "traffic": traffic},
        "cold": cold,
        "cpu_baseline": cpu,
        "achievable_hbm": achievable,
        "paths": paths,
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
