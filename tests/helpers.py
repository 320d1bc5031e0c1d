"""Shared test helpers: tensor marshalling and the error metrics."""
import numpy as np

import wkv_synth as S


def to_dev(a, bf16=False):
    """numpy -> contiguous CUDA tensor (uint16 bf16 bits become torch.bfloat16)."""
    import torch
    a = np.ascontiguousarray(a)
    if bf16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def bf16_host(t):
    """CUDA bfloat16 tensor -> exact float64 numpy array."""
    import torch
    bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return S.bf16_to_f32(bits).astype(np.float64)


def f64_host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def rel_errors(got, ref):
    """(rms_rel, max_rel): ||g - r||_2 / ||r||_2 and
    max_i |g_i - r_i| / max(|r_i|, rms(r))."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    nr = np.linalg.norm(ref)
    if nr == 0:
        return float(np.linalg.norm(got)), float(np.max(np.abs(got), initial=0.0))
    rms = nr / np.sqrt(ref.size)
    d = np.abs(got - ref)
    return float(np.linalg.norm(got - ref) / nr), float(np.max(d / np.maximum(np.abs(ref), rms)))


# tolerances for bf16-input Eagle / Finch (RMS relative, max relative)
RMS_TOL = 5e-3
MAX_TOL = 3e-2
# RWKV-4 fp32: max |y - y_ref| / max(|y_ref|, |v|-weighted average)
RWKV4_TOL = 1e-5


def assert_matrix_close(got, ref, what):
    rms, mx = rel_errors(got, ref)
    assert rms <= RMS_TOL and mx <= MAX_TOL, f"{what}: rms_rel {rms:.3e}, max_rel {mx:.3e}"
    return rms, mx


def matrix_inputs_dev(d, per_token=True):
    """Move a wkv_synth matrix-input dict to the GPU."""
    return dict(r=to_dev(d["r"], True), k=to_dev(d["k"], True), v=to_dev(d["v"], True),
                x=to_dev(d["x"]), u=to_dev(d["u"]), s0=to_dev(d["s0"]))


def matrix_inputs_f32(d):
    """The exact fp32 values the GPU sees, for the oracle."""
    return (S.bf16_to_f32(d["r"]), S.bf16_to_f32(d["k"]), S.bf16_to_f32(d["v"]),
            d["x"], d["u"], d["s0"])


def assert_heads_close(got, ref, axes, what):
    """The bf16 tolerances applied to every (sequence, head) on its own:
    `axes` are the axes of one head's elements (tokens and channels of an
    output [B, T, H, N]: (1, 3); a state [B, H, N, N]: (2, 3)).  Returns the
    worst head's (rms_rel, max_rel, index)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    n = int(np.prod([ref.shape[a] for a in axes]))
    diff = got - ref
    nr = np.sqrt(np.sum(ref * ref, axis=axes, keepdims=True))
    rms = nr / np.sqrt(n)
    with np.errstate(divide="ignore", invalid="ignore"):
        rms_rel = np.sqrt(np.sum(diff * diff, axis=axes, keepdims=True)) / nr
        max_rel = np.max(np.abs(diff) / np.maximum(np.abs(ref), rms), axis=axes, keepdims=True)
    # an all-zero reference head must come out exactly zero
    zero = nr == 0
    rms_rel = np.where(zero, np.sqrt(np.sum(diff * diff, axis=axes, keepdims=True)), rms_rel)
    max_rel = np.where(zero, np.max(np.abs(diff), axis=axes, keepdims=True), max_rel)
    rms_rel, max_rel = np.squeeze(rms_rel, axis=axes), np.squeeze(max_rel, axis=axes)
    i = np.unravel_index(int(np.argmax(rms_rel)), rms_rel.shape)
    j = np.unravel_index(int(np.argmax(max_rel)), max_rel.shape)
    assert rms_rel[i] <= RMS_TOL, f"{what}: head {i} rms_rel {rms_rel[i]:.3e}"
    assert max_rel[j] <= MAX_TOL, f"{what}: head {j} max_rel {max_rel[j]:.3e}"
    return float(rms_rel[i]), float(max_rel[j]), tuple(int(a) for a in i)


def ulp_diff(a, b):
    """Distance between two fp32 arrays in units in the last place (0 where
    bit-identical); signed zeros count as equal."""
    ia = np.ascontiguousarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.ascontiguousarray(b, np.float32).view(np.int32).astype(np.int64)
    # map the sign-magnitude bits onto a monotonic integer line
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)
