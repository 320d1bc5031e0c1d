"""RWKV WKV operators on AMD Instinct MI355X (gfx950).

Thin Python binding of ``librwkv_wkv.so``: it checks tensor shapes, dtypes and
devices, allocates missing outputs with torch, and passes raw device pointers
and the current HIP stream to the C ABI declared in ``include/rwkv_wkv.h``.
Every step of the computation runs in the library's HIP kernels; there is no
other implementation to fall back to, and calling any operator without the
built library raises.

Operators (names as in the C ABI):
  rwkv4_wkv_fwd   RWKV-4 per-channel WKV, fp32, time-parallel
  rwkv4_wkv_step  RWKV-4 per-channel WKV, fp32, serial (decode)
  rwkv5_wkv_fwd   Eagle matrix-state WKV, time-parallel (chunked)
  rwkv5_wkv_step  Eagle matrix-state WKV, serial (decode)
  rwkv6_wkv_fwd   Finch matrix-state WKV, time-parallel (chunked)
  rwkv6_wkv_step  Finch matrix-state WKV, serial (decode)
  rwkv5_wkv_fwd_gated, rwkv6_wkv_fwd_gated
                  the chunked forward with the LayerNorm-per-head and SiLU-gate
                  epilogue fused into the output
  rwkv5_wkv_bwd   Eagle backward of the chunked forward
  rwkv6_wkv_bwd   Finch backward of the chunked forward
  rwkv6_decay_lora, rwkv6_wkv_fwd_lora
                  the Finch decay producer, alone or fused into the forward
  rwkv5/6_wkv_fwd_save, rwkv5/6_wkv_bwd_saved
                  the training pair (the forward keeps the chunk states)
Entry points with device scratch take a ``workspace`` (uint8 tensor): the
caller zero-fills it once (new_workspace) and may then reuse it for any
number of calls; by default each call makes a fresh one.
"""
from __future__ import annotations

import ctypes
import os

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librwkv_wkv.so")

RWKV_OK = 0
STATUS = {0: "RWKV_OK", -1: "RWKV_E_NULL", -2: "RWKV_E_DIM", -3: "RWKV_E_UNSUPPORTED",
          -4: "RWKV_E_ALIGN", -5: "RWKV_E_ALIAS", -6: "RWKV_E_HIP", -7: "RWKV_E_TIMEOUT"}
EXPORTS = ("rwkv_wkv_strerror", "rwkv_wkv_workspace_status", "rwkv4_wkv_fwd",
           "rwkv4_wkv_fwd_workspace_bytes", "rwkv4_wkv_step", "rwkv5_wkv_fwd",
           "rwkv5_wkv_step", "rwkv6_wkv_fwd", "rwkv6_wkv_step", "rwkv_wkv_fwd_workspace_bytes",
           "rwkv5_wkv_bwd", "rwkv6_wkv_bwd", "rwkv_wkv_bwd_workspace_bytes",
           "rwkv5_wkv_fwd_gated", "rwkv6_wkv_fwd_gated", "rwkv6_decay_lora",
           "rwkv6_decay_lora_workspace_bytes", "rwkv6_wkv_fwd_lora",
           "rwkv6_wkv_fwd_lora_workspace_bytes", "rwkv5_wkv_fwd_save", "rwkv6_wkv_fwd_save",
           "rwkv5_wkv_bwd_saved", "rwkv6_wkv_bwd_saved", "rwkv6_wkv_fwd_noalloc")

_lib = None


class WKVError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({text})")
        self.status = status


def lib():
    """The loaded C library (ctypes), with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(
                f"{LIBRARY} is not built; run `python -m linear_attention_rnn_wkv_amd._build`")
        L = ctypes.CDLL(LIBRARY)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.rwkv_wkv_strerror.restype = ctypes.c_char_p
        L.rwkv_wkv_strerror.argtypes = [I]
        L.rwkv_wkv_workspace_status.restype = I
        L.rwkv_wkv_workspace_status.argtypes = [P, Z, P]
        for name in ("rwkv4_wkv_fwd_workspace_bytes", "rwkv_wkv_fwd_workspace_bytes",
                     "rwkv_wkv_bwd_workspace_bytes", "rwkv6_wkv_fwd_lora_workspace_bytes"):
            f = getattr(L, name)
            f.restype = Z
            f.argtypes = [I, I, I, I]
        L.rwkv6_decay_lora_workspace_bytes.restype = Z
        L.rwkv6_decay_lora_workspace_bytes.argtypes = [I, I, I]
        L.rwkv4_wkv_fwd.restype = I
        L.rwkv4_wkv_fwd.argtypes = [I, I, I, I, P, P, P, P, P, P, P, P, Z, P]
        for name in ("rwkv5_wkv_fwd", "rwkv6_wkv_fwd"):
            f = getattr(L, name)
            f.restype = I
            f.argtypes = [I, I, I, I, P, P, P, P, P, P, P, P, P, Z, P]
        L.rwkv6_wkv_fwd_noalloc.restype = I
        L.rwkv6_wkv_fwd_noalloc.argtypes = [I, I, I, I, P, P, P, P, P, P, P, P, P]
        L.rwkv4_wkv_step.restype = I
        L.rwkv4_wkv_step.argtypes = [I, I, I, I, P, P, P, P, P, P, P]
        for name in ("rwkv5_wkv_step", "rwkv6_wkv_step"):
            f = getattr(L, name)
            f.restype = I
            f.argtypes = [I, I, I, I, P, P, P, P, P, P, P, P]
        for name in ("rwkv5_wkv_fwd_gated", "rwkv6_wkv_fwd_gated"):
            f = getattr(L, name)
            f.restype = I
            f.argtypes = [I, I, I, I] + [P] * 10 + [ctypes.c_float, P, P, Z, P]
        for name in ("rwkv5_wkv_bwd", "rwkv6_wkv_bwd"):
            f = getattr(L, name)
            f.restype = I
            f.argtypes = [I, I, I, I] + [P] * 15 + [Z, P]
        for name in ("rwkv5_wkv_fwd_save", "rwkv6_wkv_fwd_save"):
            f = getattr(L, name)
            f.restype = I
            f.argtypes = [I, I, I, I] + [P] * 9 + [Z, P]
        for name in ("rwkv5_wkv_bwd_saved", "rwkv6_wkv_bwd_saved"):
            f = getattr(L, name)
            f.restype = I
            f.argtypes = [I, I, I, I] + [P] * 14 + [Z, P]
        L.rwkv6_decay_lora.restype = I
        L.rwkv6_decay_lora.argtypes = [I, I, I, I] + [P] * 11 + [Z, P]
        L.rwkv6_wkv_fwd_lora.restype = I
        L.rwkv6_wkv_fwd_lora.argtypes = [I, I, I, I] + [P] * 12 + [I] + [P] * 5 + [Z, P]
        _lib = L
    return _lib


def _check(fn, status):
    if status != RWKV_OK:
        raise WKVError(fn, status, lib().rwkv_wkv_strerror(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _expect(name, t, shape, dtype):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _nbytes(t):
    return 0 if t is None else t.numel()


def new_workspace(nbytes, device="cuda"):
    """A zero-filled uint8 device tensor of nbytes (None for 0): a workspace
    ready for its first use."""
    import torch
    return torch.zeros(int(nbytes), dtype=torch.uint8, device=device) if nbytes else None


def _use_workspace(workspace, need, device):
    """The caller's workspace (checked), or a fresh zero-filled one."""
    import torch
    if workspace is None:
        return new_workspace(need, device)
    if workspace.dtype != torch.uint8 or workspace.device.type != "cuda" or \
            not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
    return workspace


def workspace_status(workspace, stream=None):
    """Waits for `stream` and raises WKVError (RWKV_E_TIMEOUT) if a kernel
    that used `workspace` gave up waiting for another workgroup's hand-off
    since the last check (the affected outputs then read NaN).  Never raised
    in normal operation.  A None or too-small workspace is not checked."""
    if workspace is None or workspace.numel() < 16384:
        return
    _check("rwkv_wkv_workspace_status", lib().rwkv_wkv_workspace_status(
        _ptr(workspace), workspace.numel(), _stream(stream)))


def rwkv4_workspace_bytes(B, T, C, H=1):
    """Bytes of (zero-filled) workspace rwkv4_wkv_fwd needs (0: none)."""
    return int(lib().rwkv4_wkv_fwd_workspace_bytes(B, T, H, C // H))


def fwd_workspace_bytes(B, T, H, N=64):
    """Bytes of (zero-filled) workspace the chunked Eagle/Finch forwards and
    their gated variants need on the current device (0: none)."""
    return int(lib().rwkv_wkv_fwd_workspace_bytes(B, T, H, N))


def lora_workspace_bytes(B, T, D):
    """Bytes of workspace rwkv6_decay_lora needs."""
    return int(lib().rwkv6_decay_lora_workspace_bytes(B, T, D))


def fwd_lora_workspace_bytes(B, T, H, N=64):
    """Bytes of (zero-filled) workspace rwkv6_wkv_fwd_lora needs."""
    return int(lib().rwkv6_wkv_fwd_lora_workspace_bytes(B, T, H, N))


def rwkv4_wkv_fwd(k, v, w, u, state_in=None, state_out=None, y=None, H=1,
                  return_state=True, workspace=None, stream=None):
    """RWKV-4 WKV.  k, v: [B, T, C] fp32; w (decay rate), u: [C] fp32;
    state_in / state_out: [B, 3, C] fp32 (a, b, p); workspace: a uint8 tensor
    of at least rwkv4_workspace_bytes bytes, zero-filled before its first use
    (None: a fresh one per call).  Returns (y, state_out)."""
    import torch
    B, T, C = k.shape
    if C % H:
        raise ValueError("C must be divisible by H")
    f32 = torch.float32
    _expect("k", k, (B, T, C), f32)
    _expect("v", v, (B, T, C), f32)
    _expect("w", w, (C,), f32)
    _expect("u", u, (C,), f32)
    if state_in is not None:
        _expect("state_in", state_in, (B, 3, C), f32)
    if y is None:
        y = torch.empty((B, T, C), dtype=f32, device=k.device)
    _expect("y", y, (B, T, C), f32)
    if state_out is None and return_state:
        state_out = torch.empty((B, 3, C), dtype=f32, device=k.device)
    if state_out is not None:
        _expect("state_out", state_out, (B, 3, C), f32)
    if T > 0:
        workspace = _use_workspace(workspace, rwkv4_workspace_bytes(B, T, C, H), k.device)
    _check("rwkv4_wkv_fwd", lib().rwkv4_wkv_fwd(
        B, T, H, C // H, _ptr(k), _ptr(v), _ptr(w), _ptr(u), _ptr(state_in),
        _ptr(state_out), _ptr(y), _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return y, state_out


def rwkv4_wkv_step(k, v, w, u, state, y=None, H=1, stream=None):
    """RWKV-4 WKV, serial: k, v: [B, T, C] fp32 (T = 1 to decode); w, u: [C];
    state: [B, 3, C] fp32 (a, b, p), updated in place.  Returns y."""
    import torch
    B, T, C = k.shape
    if C % H:
        raise ValueError("C must be divisible by H")
    f32 = torch.float32
    _expect("k", k, (B, T, C), f32)
    _expect("v", v, (B, T, C), f32)
    _expect("w", w, (C,), f32)
    _expect("u", u, (C,), f32)
    _expect("state", state, (B, 3, C), f32)
    if y is None:
        y = torch.empty((B, T, C), dtype=f32, device=k.device)
    _expect("y", y, (B, T, C), f32)
    _check("rwkv4_wkv_step", lib().rwkv4_wkv_step(
        B, T, H, C // H, _ptr(k), _ptr(v), _ptr(w), _ptr(u), _ptr(state), _ptr(y),
        _stream(stream)))
    return y


def _matrix_args(r, k, v, x, u, per_token):
    import torch
    B, T, H, N = r.shape
    bf, f32 = torch.bfloat16, torch.float32
    _expect("r", r, (B, T, H, N), bf)
    _expect("k", k, (B, T, H, N), bf)
    _expect("v", v, (B, T, H, N), bf)
    _expect("x", x, (B, T, H, N) if per_token else (H, N), f32)
    _expect("u", u, (H, N), f32)
    return B, T, H, N


def _matrix_fwd(name, per_token, r, k, v, x, u, state_in, state_out, o, return_state,
                workspace, stream):
    import torch
    B, T, H, N = _matrix_args(r, k, v, x, u, per_token)
    if state_in is not None:
        _expect("state_in", state_in, (B, H, N, N), torch.float32)
    if o is None:
        o = torch.empty((B, T, H, N), dtype=torch.bfloat16, device=r.device)
    _expect("o", o, (B, T, H, N), torch.bfloat16)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device)
    if state_out is not None:
        _expect("state_out", state_out, (B, H, N, N), torch.float32)
    if T > 0:
        workspace = _use_workspace(workspace, fwd_workspace_bytes(B, T, H, N), r.device)
    _check(name, getattr(lib(), name)(
        B, T, H, N, _ptr(r), _ptr(k), _ptr(v), _ptr(x), _ptr(u), _ptr(state_in),
        _ptr(state_out), _ptr(o), _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return o, state_out


def rwkv5_wkv_fwd(r, k, v, x, u, state_in=None, state_out=None, o=None,
                  return_state=True, workspace=None, stream=None):
    """Eagle WKV, chunked.  r, k, v: [B, T, H, 64] bf16; x (decay logit omega),
    u: [H, 64] fp32; state: [B, H, 64, 64] fp32; workspace: a uint8 tensor of
    at least fwd_workspace_bytes bytes, zero-filled before its first use
    (None: a fresh one per call when one is needed).  Returns (o, state_out)."""
    return _matrix_fwd("rwkv5_wkv_fwd", False, r, k, v, x, u, state_in, state_out, o,
                       return_state, workspace, stream)


def rwkv6_wkv_fwd(r, k, v, x, u, state_in=None, state_out=None, o=None,
                  return_state=True, workspace=None, stream=None):
    """Finch WKV, chunked.  As rwkv5_wkv_fwd but x: [B, T, H, 64] fp32."""
    return _matrix_fwd("rwkv6_wkv_fwd", True, r, k, v, x, u, state_in, state_out, o,
                       return_state, workspace, stream)


def rwkv6_wkv_fwd_noalloc(r, k, v, x, u, state_in=None, state_out=None, o=None,
                          return_state=True, stream=None):
    """rwkv6_wkv_fwd with its hand-off scratch in the library's fixed device
    array instead of a workspace (for callers that cannot allocate; shapes
    needing more than 8 MiB of it raise RWKV_E_UNSUPPORTED; calls that overlap
    on one GPU race)."""
    import torch
    B, T, H, N = _matrix_args(r, k, v, x, u, True)
    if state_in is not None:
        _expect("state_in", state_in, (B, H, N, N), torch.float32)
    if o is None:
        o = torch.empty((B, T, H, N), dtype=torch.bfloat16, device=r.device)
    _expect("o", o, (B, T, H, N), torch.bfloat16)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device)
    if state_out is not None:
        _expect("state_out", state_out, (B, H, N, N), torch.float32)
    _check("rwkv6_wkv_fwd_noalloc", lib().rwkv6_wkv_fwd_noalloc(
        B, T, H, N, _ptr(r), _ptr(k), _ptr(v), _ptr(x), _ptr(u), _ptr(state_in),
        _ptr(state_out), _ptr(o), _stream(stream)))
    return o, state_out


def _matrix_step(name, per_token, r, k, v, x, u, state, o, stream):
    import torch
    B, T, H, N = _matrix_args(r, k, v, x, u, per_token)
    _expect("state", state, (B, H, N, N), torch.float32)
    if o is None:
        o = torch.empty((B, T, H, N), dtype=torch.bfloat16, device=r.device)
    _expect("o", o, (B, T, H, N), torch.bfloat16)
    _check(name, getattr(lib(), name)(
        B, T, H, N, _ptr(r), _ptr(k), _ptr(v), _ptr(x), _ptr(u), _ptr(state), _ptr(o),
        _stream(stream)))
    return o


def rwkv5_wkv_step(r, k, v, x, u, state, o=None, stream=None):
    """Eagle WKV, serial: as rwkv6_wkv_step but x (decay logit omega): [H, 64]."""
    return _matrix_step("rwkv5_wkv_step", False, r, k, v, x, u, state, o, stream)


def _matrix_fwd_gated(name, per_token, r, k, v, x, u, g, ln_w, ln_b, eps, state_in,
                      state_out, y, return_state, workspace, stream):
    import torch
    B, T, H, N = _matrix_args(r, k, v, x, u, per_token)
    bf, f32 = torch.bfloat16, torch.float32
    _expect("g", g, (B, T, H, N), bf)
    _expect("ln_w", ln_w, (H, N), f32)
    _expect("ln_b", ln_b, (H, N), f32)
    if state_in is not None:
        _expect("state_in", state_in, (B, H, N, N), f32)
    if y is None:
        y = torch.empty((B, T, H, N), dtype=bf, device=r.device)
    _expect("y", y, (B, T, H, N), bf)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, N, N), dtype=f32, device=r.device)
    if state_out is not None:
        _expect("state_out", state_out, (B, H, N, N), f32)
    if T > 0:
        workspace = _use_workspace(workspace, fwd_workspace_bytes(B, T, H, N), r.device)
    _check(name, getattr(lib(), name)(
        B, T, H, N, _ptr(r), _ptr(k), _ptr(v), _ptr(x), _ptr(u), _ptr(state_in),
        _ptr(state_out), _ptr(g), _ptr(ln_w), _ptr(ln_b), float(eps), _ptr(y),
        _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return y, state_out


def rwkv5_wkv_fwd_gated(r, k, v, x, u, g, ln_w, ln_b, eps=1e-5, state_in=None,
                        state_out=None, y=None, return_state=True, workspace=None,
                        stream=None):
    """Eagle forward with the epilogue: y = (LayerNorm per head of o, times
    ln_w plus ln_b) * silu(g).  g: [B, T, H, 64] bf16; ln_w, ln_b: [H, 64]
    fp32.  Returns (y, state_out)."""
    return _matrix_fwd_gated("rwkv5_wkv_fwd_gated", False, r, k, v, x, u, g, ln_w, ln_b, eps,
                             state_in, state_out, y, return_state, workspace, stream)


def rwkv6_wkv_fwd_gated(r, k, v, x, u, g, ln_w, ln_b, eps=1e-5, state_in=None,
                        state_out=None, y=None, return_state=True, workspace=None,
                        stream=None):
    """Finch forward with the epilogue (as rwkv5_wkv_fwd_gated, x per token)."""
    return _matrix_fwd_gated("rwkv6_wkv_fwd_gated", True, r, k, v, x, u, g, ln_w, ln_b, eps,
                             state_in, state_out, y, return_state, workspace, stream)


def rwkv6_wkv_step(r, k, v, x, u, state, o=None, stream=None):
    """Finch WKV, serial: r, k, v: [B, T, H, 64] bf16 (T = 1 to decode);
    x: [B, T, H, 64] fp32; u: [H, 64]; state: [B, H, 64, 64] fp32, updated in
    place.  Returns o."""
    return _matrix_step("rwkv6_wkv_step", True, r, k, v, x, u, state, o, stream)


def _matrix_bwd(name, per_token, r, k, v, x, u, d_o, state_in, d_state_out, grads,
                workspace, stream, saved=False):
    import torch
    B, T, H, N = _matrix_args(r, k, v, x, u, per_token)
    bf, f32 = torch.bfloat16, torch.float32
    _expect("d_o", d_o, (B, T, H, N), bf)
    if state_in is not None:
        _expect("state_in", state_in, (B, H, N, N), f32)
    if d_state_out is not None:
        _expect("d_state_out", d_state_out, (B, H, N, N), f32)
    g = dict(grads or {})
    dev = r.device
    g.setdefault("d_r", torch.empty((B, T, H, N), dtype=bf, device=dev))
    g.setdefault("d_k", torch.empty((B, T, H, N), dtype=bf, device=dev))
    g.setdefault("d_v", torch.empty((B, T, H, N), dtype=bf, device=dev))
    g.setdefault("d_x", torch.empty((B, T, H, N) if per_token else (H, N), dtype=f32,
                                    device=dev))
    g.setdefault("d_u", torch.empty((H, N), dtype=f32, device=dev))
    g.setdefault("d_state_in", torch.empty((B, H, N, N), dtype=f32, device=dev))
    for n, shape, dt in (("d_r", (B, T, H, N), bf), ("d_k", (B, T, H, N), bf),
                         ("d_v", (B, T, H, N), bf),
                         ("d_x", (B, T, H, N) if per_token else (H, N), f32),
                         ("d_u", (H, N), f32)):
        _expect(n, g[n], shape, dt)
    if g["d_state_in"] is not None:
        _expect("d_state_in", g["d_state_in"], (B, H, N, N), f32)
    workspace = _workspace(workspace, B, T, H, N, dev, required=saved)
    head = [_ptr(r), _ptr(k), _ptr(v), _ptr(x), _ptr(u)] + ([] if saved else [_ptr(state_in)])
    _check(name, getattr(lib(), name)(
        B, T, H, N, *head, _ptr(d_o), _ptr(d_state_out), _ptr(g["d_r"]), _ptr(g["d_k"]),
        _ptr(g["d_v"]), _ptr(g["d_x"]), _ptr(g["d_u"]), _ptr(g["d_state_in"]),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return g


def _workspace(workspace, B, T, H, N, dev, required=False):
    import torch
    if workspace is None:
        if required:
            raise ValueError("workspace is required (it holds the forward's saved states)")
        return new_workspace(lib().rwkv_wkv_bwd_workspace_bytes(B, max(T, 1), H, N), dev)
    if workspace.dtype != torch.uint8 or workspace.device.type != "cuda" or \
            not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
    return workspace


def rwkv5_wkv_bwd(r, k, v, x, u, d_o, state_in=None, d_state_out=None, grads=None,
                  workspace=None, stream=None):
    """Eagle backward.  Forward inputs as in rwkv5_wkv_fwd; d_o: [B, T, H, 64]
    bf16; d_state_out: [B, H, 64, 64] fp32 or None.  Returns a dict d_r, d_k,
    d_v (bf16), d_x ([H, 64], summed), d_u ([H, 64]), d_state_in.  ``grads``
    may supply any of the output tensors; ``workspace`` a uint8 tensor of at
    least workspace_bytes(B, T, H) bytes, zero-filled before its first use
    (None: a fresh one per call)."""
    return _matrix_bwd("rwkv5_wkv_bwd", False, r, k, v, x, u, d_o, state_in, d_state_out,
                       grads, workspace, stream)


def rwkv6_wkv_bwd(r, k, v, x, u, d_o, state_in=None, d_state_out=None, grads=None,
                  workspace=None, stream=None):
    """Finch backward: as rwkv5_wkv_bwd, with d_x [B, T, H, 64]."""
    return _matrix_bwd("rwkv6_wkv_bwd", True, r, k, v, x, u, d_o, state_in, d_state_out,
                       grads, workspace, stream)


def _matrix_fwd_save(name, per_token, r, k, v, x, u, workspace, state_in, state_out, o,
                     return_state, stream):
    import torch
    B, T, H, N = _matrix_args(r, k, v, x, u, per_token)
    if state_in is not None:
        _expect("state_in", state_in, (B, H, N, N), torch.float32)
    if o is None:
        o = torch.empty((B, T, H, N), dtype=torch.bfloat16, device=r.device)
    _expect("o", o, (B, T, H, N), torch.bfloat16)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device)
    if state_out is not None:
        _expect("state_out", state_out, (B, H, N, N), torch.float32)
    workspace = _workspace(workspace, B, T, H, N, r.device, required=True)
    _check(name, getattr(lib(), name)(
        B, T, H, N, _ptr(r), _ptr(k), _ptr(v), _ptr(x), _ptr(u), _ptr(state_in),
        _ptr(state_out), _ptr(o), _ptr(workspace), workspace.numel(), _stream(stream)))
    return o, state_out


def rwkv5_wkv_fwd_save(r, k, v, x, u, workspace, state_in=None, state_out=None, o=None,
                       return_state=True, stream=None):
    """rwkv5_wkv_fwd that also leaves in ``workspace`` (uint8, at least
    workspace_bytes(B, T, H), zero-filled before its first use) the states
    rwkv5_wkv_bwd_saved reads."""
    return _matrix_fwd_save("rwkv5_wkv_fwd_save", False, r, k, v, x, u, workspace, state_in,
                            state_out, o, return_state, stream)


def rwkv6_wkv_fwd_save(r, k, v, x, u, workspace, state_in=None, state_out=None, o=None,
                       return_state=True, stream=None):
    """rwkv6_wkv_fwd that also leaves in ``workspace`` the states
    rwkv6_wkv_bwd_saved reads."""
    return _matrix_fwd_save("rwkv6_wkv_fwd_save", True, r, k, v, x, u, workspace, state_in,
                            state_out, o, return_state, stream)


def rwkv5_wkv_bwd_saved(r, k, v, x, u, d_o, workspace, d_state_out=None, grads=None,
                        stream=None):
    """rwkv5_wkv_bwd after rwkv5_wkv_fwd_save on the same inputs and
    ``workspace``: the states it saved replace the backward's recomputation."""
    return _matrix_bwd("rwkv5_wkv_bwd_saved", False, r, k, v, x, u, d_o, None, d_state_out,
                       grads, workspace, stream, saved=True)


def rwkv6_wkv_bwd_saved(r, k, v, x, u, d_o, workspace, d_state_out=None, grads=None,
                        stream=None):
    """rwkv6_wkv_bwd after rwkv6_wkv_fwd_save (as rwkv5_wkv_bwd_saved)."""
    return _matrix_bwd("rwkv6_wkv_bwd_saved", True, r, k, v, x, u, d_o, None, d_state_out,
                       grads, workspace, stream, saved=True)


def workspace_bytes(B, T, H, N=64):
    """Bytes of (zero-filled) device workspace the backward, and the forward
    and backward of the training pair, need on the current device."""
    return int(lib().rwkv_wkv_bwd_workspace_bytes(B, T, H, N))


ACTS = {"identity": 0, "tanh": 1}


def _lora_args(x, shift, mu_x, lam, A1, B1, omega, A2, B2, act):
    import torch
    B, T, D = x.shape
    bf, f32 = torch.bfloat16, torch.float32
    _expect("x", x, (B, T, D), bf)
    if shift is not None:
        _expect("shift", shift, (B, D), bf)
    for name, t in (("mu_x", mu_x), ("lam", lam), ("omega", omega)):
        _expect(name, t, (D,), f32)
    _expect("A1", A1, (D, 32), bf)
    _expect("B1", B1, (32, D), bf)
    _expect("A2", A2, (D, 64), bf)
    _expect("B2", B2, (64, D), bf)
    if act not in ACTS:
        raise ValueError(f"act must be one of {sorted(ACTS)}")
    return B, T, D


def rwkv6_decay_lora(x, mu_x, lam, A1, B1, omega, A2, B2, act="tanh", shift=None, d=None,
                     workspace=None, stream=None):
    """Finch decay logits d [B, T, D] fp32 from the block input x [B, T, D]
    bf16: ddlerp with the mix's LoRA (A1 [D, 32], B1 [32, D] bf16, mu_x and
    lam [D] fp32), then LoRA_omega (A2 [D, 64], B2 [64, D] bf16, omega [D]);
    act "tanh" or "identity"; shift [B, D] bf16, the token before x[:, 0]
    (None = zeros)."""
    import torch
    B, T, D = _lora_args(x, shift, mu_x, lam, A1, B1, omega, A2, B2, act)
    if d is None:
        d = torch.empty((B, T, D), dtype=torch.float32, device=x.device)
    _expect("d", d, (B, T, D), torch.float32)
    if T > 0 and workspace is None:
        workspace = torch.empty(lora_workspace_bytes(B, T, D), dtype=torch.uint8,
                                device=x.device)
    workspace = _use_workspace(workspace, 0, x.device)
    _check("rwkv6_decay_lora", lib().rwkv6_decay_lora(
        B, T, D, ACTS[act], _ptr(x), _ptr(shift), _ptr(mu_x), _ptr(lam), _ptr(A1), _ptr(B1),
        _ptr(omega), _ptr(A2), _ptr(B2), _ptr(d), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))
    return d


def rwkv6_wkv_fwd_lora(r, k, v, x, mu_x, lam, A1, B1, omega, A2, B2, u, act="tanh",
                       shift=None, state_in=None, state_out=None, o=None, return_state=True,
                       workspace=None, stream=None):
    """Finch WKV, chunked, with the decay logits made on the device from the
    block input x [B, T, H*64] bf16 (as rwkv6_decay_lora): the result of
    rwkv6_wkv_fwd(r, k, v, rwkv6_decay_lora(...).view(B, T, H, 64), u, ...)."""
    import torch
    B, T, H, N = r.shape
    bf, f32 = torch.bfloat16, torch.float32
    for name, t in (("r", r), ("k", k), ("v", v)):
        _expect(name, t, (B, T, H, N), bf)
    _expect("u", u, (H, N), f32)
    _expect("x", x, (B, T, H * N), bf)
    _lora_args(x, shift, mu_x, lam, A1, B1, omega, A2, B2, act)
    if state_in is not None:
        _expect("state_in", state_in, (B, H, N, N), f32)
    if o is None:
        o = torch.empty((B, T, H, N), dtype=bf, device=r.device)
    _expect("o", o, (B, T, H, N), bf)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, N, N), dtype=f32, device=r.device)
    if state_out is not None:
        _expect("state_out", state_out, (B, H, N, N), f32)
    if T > 0:
        workspace = _use_workspace(workspace, fwd_lora_workspace_bytes(B, T, H, N), r.device)
    _check("rwkv6_wkv_fwd_lora", lib().rwkv6_wkv_fwd_lora(
        B, T, H, N, _ptr(r), _ptr(k), _ptr(v), _ptr(x), _ptr(shift), _ptr(mu_x), _ptr(lam),
        _ptr(A1), _ptr(B1), _ptr(omega), _ptr(A2), _ptr(B2), ACTS[act], _ptr(u),
        _ptr(state_in), _ptr(state_out), _ptr(o), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))
    return o, state_out
