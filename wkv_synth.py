"""Seeded synthetic inputs for the WKV operators.

This module holds no part of the WKV arithmetic: it only draws random numbers
and rounds them to the storage types the operators take (fp32, or bf16 kept
as raw uint16 bits).  Both the oracle side and the GPU side of every test and
benchmark consume the same rounded values.

Generation is blocked: a tensor is cut into fixed blocks of ``BLOCK``
elements and block ``i`` of tensor ``tid`` for workload ``cfg`` is drawn from
``PCG64(SeedSequence([cfg, tid, i]))``.  The values therefore depend only on
(cfg, tid, shape), never on the thread count used to draw them.

Distributions follow the workloads the pages' model widths suggest (see
``workload``); "N(0, s)" means standard deviation s.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK = 1 << 20

# tensor ids (stable: changing one changes every stored expectation)
T_R, T_K, T_V, T_OMEGA, T_DELTA, T_U, T_S0, T_W = 1, 2, 3, 4, 5, 6, 7, 4
T_DO, T_DST = 8, 9  # gradients arriving at the backward
T_G, T_LNW, T_LNB = 10, 11, 12  # gate and norm parameters of the output epilogue
# the Finch decay producer's block input, shift row and parameters
T_XIN, T_SHIFT, T_MUX, T_LAM, T_A1, T_B1, T_A2, T_B2 = 13, 14, 15, 16, 17, 18, 19, 20


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill(shape, cfg, tid, draw):
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, np.float32)
    nblocks = (n + BLOCK - 1) // BLOCK

    def one(i):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, tid, i])))
        seg = out[i * BLOCK:min(n, (i + 1) * BLOCK)]
        draw(g, seg)

    if nblocks <= 1:
        for i in range(nblocks):
            one(i)
    else:
        with ThreadPoolExecutor(min(_threads(), nblocks)) as ex:
            list(ex.map(one, range(nblocks)))
    return out.reshape(shape)


def normal(shape, sigma, cfg, tid, mean=0.0):
    """fp32 array of N(mean, sigma) draws."""
    def draw(g, seg):
        g.standard_normal(out=seg, dtype=np.float32)
        if sigma != 1.0:
            seg *= np.float32(sigma)
        if mean != 0.0:
            seg += np.float32(mean)
    return _fill(shape, cfg, tid, draw)


def uniform(shape, lo, hi, cfg, tid):
    """fp32 array of U(lo, hi) draws."""
    def draw(g, seg):
        g.random(out=seg, dtype=np.float32)
        seg *= np.float32(hi - lo)
        seg += np.float32(lo)
    return _fill(shape, cfg, tid, draw)


def to_bf16(a):
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bits = bits + 0x7FFF + ((bits >> 16) & 1)
    return (bits >> 16).astype(np.uint16).reshape(a.shape)


def bf16_to_f32(bits):
    """Exact widening of bf16 bits (uint16) to fp32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).reshape(bits.shape)


# ---------------------------------------------------------------------------
# operator inputs

def rwkv4_inputs(B, T, C, cfg, k_sigma=1.0):
    """RWKV-4: k, v [B,T,C] fp32; w ~ U(0.01, 5), u ~ N(0, 0.5) per channel."""
    return {
        "k": normal((B, T, C), k_sigma, cfg, T_K),
        "v": normal((B, T, C), 1.0, cfg, T_V),
        "w": uniform((C,), 0.01, 5.0, cfg, T_W),
        "u": normal((C,), 0.5, cfg, T_U),
    }


def wkv_inputs(B, T, H, N, cfg, per_token, s0_sigma=0.0, rkv_sigma=0.125,
               omega=(-6.0, -0.5), delta_sigma=0.5, u_sigma=0.5):
    """Eagle (per_token=False) / Finch (per_token=True) inputs.

    r, k, v: bf16 bits [B,T,H,N] ~ N(0, rkv_sigma); omega ~ U(omega) [H,N];
    Finch: x = omega + delta, delta ~ N(0, delta_sigma) iid [B,T,H,N] fp32;
    Eagle: x = omega [H,N]; u ~ N(0, u_sigma) [H,N];
    s0: fp32 [B,H,N,N] ~ N(0, s0_sigma) (zeros when s0_sigma == 0).
    """
    d = {
        "r": to_bf16(normal((B, T, H, N), rkv_sigma, cfg, T_R)),
        "k": to_bf16(normal((B, T, H, N), rkv_sigma, cfg, T_K)),
        "v": to_bf16(normal((B, T, H, N), rkv_sigma, cfg, T_V)),
        "u": normal((H, N), u_sigma, cfg, T_U),
    }
    om = uniform((H, N), omega[0], omega[1], cfg, T_OMEGA)
    if per_token:
        x = normal((B, T, H, N), delta_sigma, cfg, T_DELTA)
        x += om  # broadcast over (B, T)
        d["x"] = x
    else:
        d["x"] = om
    if s0_sigma > 0:
        d["s0"] = normal((B, H, N, N), s0_sigma, cfg, T_S0)
    else:
        d["s0"] = np.zeros((B, H, N, N), np.float32)
    return d


def grad_inputs(B, T, H, N, cfg, do_sigma=0.125, dst_sigma=0.1):
    """Gradients arriving at the backward: d_o bf16 bits [B,T,H,N] ~
    N(0, do_sigma); d_sT fp32 [B,H,N,N] ~ N(0, dst_sigma) (zeros when 0)."""
    d = {"d_o": to_bf16(normal((B, T, H, N), do_sigma, cfg, T_DO))}
    d["d_sT"] = (normal((B, H, N, N), dst_sigma, cfg, T_DST) if dst_sigma > 0
                 else np.zeros((B, H, N, N), np.float32))
    return d


def epilogue_inputs(B, T, H, N, cfg, g_sigma=1.0, w_sigma=0.1, b_sigma=0.1):
    """Output epilogue: gate g bf16 bits [B,T,H,N] ~ N(0, g_sigma); norm
    weight ln_w ~ 1 + N(0, w_sigma) and bias ln_b ~ N(0, b_sigma), fp32 [H,N]."""
    return {"g": to_bf16(normal((B, T, H, N), g_sigma, cfg, T_G)),
            "ln_w": normal((H, N), w_sigma, cfg, T_LNW, mean=1.0),
            "ln_b": normal((H, N), b_sigma, cfg, T_LNB)}


def decay_lora_inputs(B, T, H, N, cfg, omega=(-6.0, -0.5), shift=True, b1_sigma=0.05,
                      b2_sigma=0.1):
    """Finch decay producer: block input x bf16 bits [B,T,H N] ~ N(0, 1) (a
    LayerNorm output); shift row bf16 [B, H N] ~ N(0, 1) (None when shift is
    False); mu_x, lam ~ U(0, 1) fp32 [H N]; A1 [H N, 32] and A2 [H N, 64] bf16
    ~ N(0, 1/sqrt(H N)), so that the LoRA inputs' products are of order one;
    B1 [32, H N] ~ N(0, b1_sigma), B2 [64, H N] ~ N(0, b2_sigma) bf16; omega
    ~ U(omega) fp32 [H N].  Under tanh the logit offset act(z A2) B2 then
    spreads like the Finch workload's delta (RMS about 0.5)."""
    D = H * N
    a_sigma = 1.0 / np.sqrt(D)
    return {
        "xin": to_bf16(normal((B, T, D), 1.0, cfg, T_XIN)),
        "shift": to_bf16(normal((B, D), 1.0, cfg, T_SHIFT)) if shift else None,
        "mu_x": uniform((D,), 0.0, 1.0, cfg, T_MUX),
        "lam": uniform((D,), 0.0, 1.0, cfg, T_LAM),
        "A1": to_bf16(normal((D, 32), a_sigma, cfg, T_A1)),
        "B1": to_bf16(normal((32, D), b1_sigma, cfg, T_B1)),
        "omega": uniform((D,), omega[0], omega[1], cfg, T_OMEGA),
        "A2": to_bf16(normal((D, 64), a_sigma, cfg, T_A2)),
        "B2": to_bf16(normal((64, D), b2_sigma, cfg, T_B2)),
    }


def decode_inputs(B, steps, H, N, cfg, s0_sigma=0.1, rkv_sigma=0.125,
                  omega=(-6.0, -0.5), delta_sigma=0.5, u_sigma=0.5, per_token=True):
    """Finch (Eagle: per_token=False) decode: per-step r, k, v (bf16 bits) and
    Finch's x (fp32) laid out [steps][B][H][N] so that each step's slice is one
    contiguous [B,1,H,N] operand; Eagle's x [H,N]; u [H,N]; s0 [B,H,N,N]."""
    d = wkv_inputs(steps, B, H, N, cfg, per_token, 0.0, rkv_sigma, omega,
                   delta_sigma, u_sigma)
    d["s0"] = (normal((B, H, N, N), s0_sigma, cfg, T_S0) if s0_sigma > 0
               else np.zeros((B, H, N, N), np.float32))
    return d


# ---------------------------------------------------------------------------
# the named workloads

WORKLOADS = {
    1: dict(kind="rwkv4", B=1, T=64, C=64, k_sigma=1.0),
    2: dict(kind="rwkv4", B=8, T=1024, C=768, k_sigma=2.0),
    3: dict(kind="eagle", B=8, T=4096, H=32, N=64, s0_sigma=0.0),
    4: dict(kind="finch", B=8, T=4096, H=40, N=64, s0_sigma=0.1),
    5: dict(kind="decode", B=256, steps=1024, H=64, N=64, s0_sigma=0.1),
    # serial mode of the other two generations at the same 7B-class width
    6: dict(kind="eagle_decode", B=256, steps=1024, H=64, N=64, s0_sigma=0.1),
    7: dict(kind="rwkv4_decode", B=256, steps=1024, C=4096, k_sigma=2.0),
}

WORKLOAD_NAMES = {
    1: "rwkv4_fwd_B1_T64_C64_fp32",
    2: "rwkv4_fwd_B8_T1024_C768_fp32",
    3: "eagle_fwd_B8_T4096_D2048_H32_N64_bf16",
    4: "finch_fwd_B8_T4096_D2560_H40_N64_bf16",
    5: "finch_decode_B256_D4096_H64_N64_x1024",
    6: "eagle_decode_B256_D4096_H64_N64_x1024",
    7: "rwkv4_decode_B256_C4096_x1024",
}


def workload(cfg, **override):
    """Inputs of workload ``cfg`` (1..7); keyword overrides change sizes."""
    spec = dict(WORKLOADS[cfg])
    spec.update(override)
    kind = spec.pop("kind")
    if kind == "rwkv4":
        return rwkv4_inputs(spec["B"], spec["T"], spec["C"], cfg, spec["k_sigma"])
    if kind == "eagle":
        return wkv_inputs(spec["B"], spec["T"], spec["H"], spec["N"], cfg, False,
                          spec["s0_sigma"])
    if kind == "finch":
        return wkv_inputs(spec["B"], spec["T"], spec["H"], spec["N"], cfg, True,
                          spec["s0_sigma"])
    if kind in ("decode", "eagle_decode"):
        return decode_inputs(spec["B"], spec["steps"], spec["H"], spec["N"], cfg,
                             spec["s0_sigma"], per_token=kind == "decode")
    if kind == "rwkv4_decode":
        # k, v [steps][B][C]: each step's slice is one contiguous [B,1,C] operand
        return rwkv4_inputs(spec["steps"], spec["B"], spec["C"], cfg, spec["k_sigma"])
    raise ValueError(kind)
