"""fp64 CPU oracle for the RWKV WKV recurrence (RWKV-4, Eagle, Finch).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The HIP library never imports, links
or runs anything in this directory, and this directory never touches the HIP
library.

The arithmetic lives in ``wkv_oracle.c`` (plain C, double precision, one token
at a time); this module only compiles it with gcc and marshals numpy arrays
through ctypes.  See the header of ``wkv_oracle.c`` for the definitions and
the passages of the pages they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "wkv_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc.  No fast-math, no FMA contraction."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-shared", "-fPIC", "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def _bind(lib):
    d = ctypes.POINTER(ctypes.c_double)
    f = ctypes.POINTER(ctypes.c_float)
    L = ctypes.c_long
    lib.oracle_rwkv4_fwd.restype = ctypes.c_int
    lib.oracle_rwkv4_fwd.argtypes = [L, L, L, f, f, f, f, d, d, d, d, d, d,
                                     ctypes.c_int]
    lib.oracle_wkv_matrix.restype = ctypes.c_int
    lib.oracle_wkv_matrix.argtypes = [L, L, L, L, f, f, f, f, ctypes.c_int, f,
                                      d, d, d, ctypes.c_int]
    lib.oracle_norm_gate.restype = ctypes.c_int
    lib.oracle_norm_gate.argtypes = [L, L, L, d, f, f, f, ctypes.c_double, d, ctypes.c_int]
    lib.oracle_decay_lora.restype = ctypes.c_int
    lib.oracle_decay_lora.argtypes = [L, L, L, L, L, f, f, f, f, f, f, f, f, f, ctypes.c_int, d,
                                      ctypes.c_int]
    lib.oracle_wkv_matrix_bwd.restype = ctypes.c_int
    lib.oracle_wkv_matrix_bwd.argtypes = [L, L, L, L, f, f, f, f, ctypes.c_int, f,
                                          d, d, d, d, d, d, d, d, d, ctypes.c_int]
    return lib


def load(path: str | None = None):
    """Load the compiled oracle, building it first if it is missing."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIBRARY) or (
                os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
            build()
        _lib = _bind(ctypes.CDLL(LIBRARY))
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _null_d():
    return ctypes.POINTER(ctypes.c_double)()


def rwkv4_fwd(k, v, w, u, num_in=None, den_in=None, nthreads=None, lib=None):
    """RWKV-4 WKV in fp64.

    k, v: [B, T, C]; w, u: [C]; num_in, den_in: [B, C] history (None = empty).
    Returns a dict with y, scale ([B, T, C]) and num, den ([B, C]), all float64.
    """
    lib = lib or load()
    k, kp = _f32(k)
    v, vp = _f32(v)
    w, wp = _f32(w)
    u, up = _f32(u)
    B, T, C = k.shape
    assert v.shape == k.shape and w.shape == (C,) and u.shape == (C,)
    keep = []
    if num_in is None:
        nip, dip = _null_d(), _null_d()
    else:
        ni, nip = _f64(num_in)
        di, dip = _f64(den_in)
        assert ni.shape == (B, C) and di.shape == (B, C)
        keep += [ni, di]
    y = np.empty((B, T, C), np.float64)
    scale = np.empty((B, T, C), np.float64)
    num = np.empty((B, C), np.float64)
    den = np.empty((B, C), np.float64)
    rc = lib.oracle_rwkv4_fwd(B, T, C, kp, vp, wp, up, nip, dip,
                              _f64(y)[1], _f64(scale)[1], _f64(num)[1],
                              _f64(den)[1], int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_rwkv4_fwd failed ({rc})")
    return {"y": y, "scale": scale, "num": num, "den": den}


def wkv_matrix(r, k, v, x, u, s_in=None, nthreads=None, lib=None):
    """Eagle / Finch WKV in fp64.

    r, k, v: [B, T, H, N]; x: [H, N] (Eagle, static decay logit) or
    [B, T, H, N] (Finch, per-token logit); u: [H, N];
    s_in: [B, H, N, N] (None = zeros).
    Returns (o [B, T, H, N], s_out [B, H, N, N]), float64.
    """
    lib = lib or load()
    r, rp = _f32(r)
    k, kp = _f32(k)
    v, vp = _f32(v)
    x, xp = _f32(x)
    u, up = _f32(u)
    B, T, H, N = r.shape
    assert k.shape == r.shape and v.shape == r.shape and u.shape == (H, N)
    if x.shape == (H, N):
        per_token = 0
    else:
        assert x.shape == r.shape, x.shape
        per_token = 1
    if s_in is None:
        sp = _null_d()
    else:
        s_in, sp = _f64(s_in)
        assert s_in.shape == (B, H, N, N)
    o = np.empty((B, T, H, N), np.float64)
    s_out = np.empty((B, H, N, N), np.float64)
    rc = lib.oracle_wkv_matrix(B, T, H, N, rp, kp, vp, xp, per_token, up, sp,
                               _f64(o)[1], _f64(s_out)[1],
                               int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_wkv_matrix failed ({rc})")
    return o, s_out


def wkv_matrix_bwd(r, k, v, x, u, d_o, s_in=None, d_sT=None, nthreads=None, lib=None):
    """Eagle / Finch WKV backward in fp64 (reverse-mode of the serial
    recurrence).

    Forward inputs as in wkv_matrix; d_o: [B, T, H, N] gradient of the output;
    d_sT: [B, H, N, N] gradient of the final state (None = zero).
    Returns a dict of float64 arrays: dr, dk, dv ([B, T, H, N]), dx
    ([B, T, H, N] for Finch, [H, N] summed over b and t for Eagle), du ([H, N],
    summed over b and t) and ds0 ([B, H, N, N]).
    """
    lib = lib or load()
    r, rp = _f32(r)
    k, kp = _f32(k)
    v, vp = _f32(v)
    x, xp = _f32(x)
    u, up = _f32(u)
    B, T, H, N = r.shape
    assert k.shape == r.shape and v.shape == r.shape and u.shape == (H, N)
    per_token = 0 if x.shape == (H, N) else 1
    if per_token:
        assert x.shape == r.shape, x.shape
    keep = []
    if s_in is None:
        sp = _null_d()
    else:
        s_in, sp = _f64(s_in)
        assert s_in.shape == (B, H, N, N)
    d_o, dop = _f64(d_o)
    assert d_o.shape == r.shape
    if d_sT is None:
        dsp = _null_d()
    else:
        d_sT, dsp = _f64(d_sT)
        assert d_sT.shape == (B, H, N, N)
    out = {n: np.empty(r.shape, np.float64) for n in ("dr", "dk", "dv")}
    out["dx"] = np.empty(r.shape if per_token else (H, N), np.float64)
    out["du"] = np.empty((H, N), np.float64)
    out["ds0"] = np.empty((B, H, N, N), np.float64)
    rc = lib.oracle_wkv_matrix_bwd(B, T, H, N, rp, kp, vp, xp, per_token, up, sp, dop, dsp,
                                   _f64(out["dr"])[1], _f64(out["dk"])[1], _f64(out["dv"])[1],
                                   _f64(out["dx"])[1], _f64(out["du"])[1],
                                   _f64(out["ds0"])[1], int(nthreads or default_threads()))
    del keep
    if rc != 0:
        raise RuntimeError(f"oracle_wkv_matrix_bwd failed ({rc})")
    return out


def norm_gate(o, g, ln_w, ln_b, eps, nthreads=None, lib=None):
    """Eagle / Finch output epilogue in fp64: per head and token, LayerNorm of
    o over the head's channels (eps added to the biased variance), times ln_w
    plus ln_b, times silu(g).  o, g: [..., H, N]; ln_w, ln_b: [H, N]."""
    lib = lib or load()
    o, op = _f64(o)
    g, gp = _f32(g)
    ln_w, wp = _f32(ln_w)
    ln_b, bp = _f32(ln_b)
    H, N = o.shape[-2:]
    assert g.shape == o.shape and ln_w.shape == (H, N) and ln_b.shape == (H, N)
    rows = o.size // (H * N)
    y = np.empty(o.shape, np.float64)
    rc = lib.oracle_norm_gate(rows, H, N, op, gp, wp, bp, float(eps), _f64(y)[1],
                              int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_norm_gate failed ({rc})")
    return y


def decay_lora(x, mu_x, lam, A1, B1, omega, A2, B2, act="tanh", shift=None, nthreads=None,
               lib=None):
    """Finch decay logits d [B, T, D] (float64) from the block input x
    [B, T, D] by ddlerp and LoRA_omega (see oracle_decay_lora).

    mu_x, lam, omega: [D]; A1: [D, R1]; B1: [R1, D]; A2: [D, R2]; B2: [R2, D];
    act: "identity" or "tanh"; shift: [B, D], the token before x[:, 0]
    (None = zeros)."""
    lib = lib or load()
    x, xp = _f32(x)
    B, T, D = x.shape
    mu_x, mup = _f32(mu_x)
    lam, lp = _f32(lam)
    omega, op = _f32(omega)
    A1, a1p = _f32(A1)
    B1, b1p = _f32(B1)
    A2, a2p = _f32(A2)
    B2, b2p = _f32(B2)
    R1, R2 = A1.shape[1], A2.shape[1]
    assert mu_x.shape == (D,) and lam.shape == (D,) and omega.shape == (D,)
    assert A1.shape == (D, R1) and B1.shape == (R1, D)
    assert A2.shape == (D, R2) and B2.shape == (R2, D)
    if shift is None:
        sp = ctypes.POINTER(ctypes.c_float)()
    else:
        shift, sp = _f32(shift)
        assert shift.shape == (B, D)
    code = {"identity": 0, "tanh": 1}[act]
    d = np.empty((B, T, D), np.float64)
    rc = lib.oracle_decay_lora(B, T, D, R1, R2, xp, sp, mup, lp, a1p, b1p, op, a2p, b2p, code,
                               _f64(d)[1], int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_decay_lora failed ({rc})")
    return d
