"""The C-ABI library on the host: it loads, exports every function the header
declares, and rejects invalid arguments before any HIP call (so these run
without a GPU; dummy host addresses are never dereferenced)."""
import ctypes
import os
import re

import pytest

import linear_attention_rnn_wkv_amd as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, E_NULL, E_DIM, E_UNSUP, E_ALIGN, E_ALIAS = 0, -1, -2, -3, -4, -5


def header_functions():
    src = open(os.path.join(ROOT, "include", "rwkv_wkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rwkv\w*)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(W.LIBRARY):
        from linear_attention_rnn_wkv_amd import _build
        _build.build()
    return W.lib()


def test_header_declares_the_operators():
    assert header_functions() == sorted(W.EXPORTS)


def test_library_exports_every_declared_function(L):
    out = os.popen(f"nm -D --defined-only {W.LIBRARY}").read()
    exported = set(re.findall(r"\bT (\w+)", out))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(L, name)


def test_strerror_covers_every_status(L):
    for st in W.STATUS:
        assert L.rwkv_wkv_strerror(st).decode() != "unknown status"
    assert L.rwkv_wkv_strerror(42).decode() == "unknown status"


# fake, aligned host addresses: validation fails before they could be used
BASE = 1 << 40
SPAN = 1 << 30


def addr(i, misalign=0):
    return ctypes.c_void_p(BASE + i * SPAN + misalign)


def rwkv4(L, B=2, T=8, H=1, N=16, k=1, v=2, w=3, u=4, si=5, so=6, y=7, ws=8, ws_bytes=None,
          **mis):
    a = {n: (addr(i, mis.get(n, 0)) if i is not None else None)
         for n, i in dict(k=k, v=v, w=w, u=u, si=si, so=so, y=y, ws=ws).items()}
    if ws_bytes is None:
        ws_bytes = L.rwkv4_wkv_fwd_workspace_bytes(B, T, H, N)
    return L.rwkv4_wkv_fwd(B, T, H, N, a["k"], a["v"], a["w"], a["u"], a["si"], a["so"],
                           a["y"], a["ws"], ws_bytes, None)


def matrix(L, fn, B=2, T=8, H=2, N=64, r=1, k=2, v=3, x=4, u=5, si=6, so=7, o=8, ws=9,
           ws_bytes=None, **mis):
    a = {n: (addr(i, mis.get(n, 0)) if i is not None else None)
         for n, i in dict(r=r, k=k, v=v, x=x, u=u, si=si, so=so, o=o, ws=ws).items()}
    if ws_bytes is None:
        ws_bytes = L.rwkv_wkv_fwd_workspace_bytes(B, T, H, N)
    return getattr(L, fn)(B, T, H, N, a["r"], a["k"], a["v"], a["x"], a["u"], a["si"],
                          a["so"], a["o"], a["ws"], ws_bytes, None)


def step(L, B=2, T=1, H=2, N=64, r=1, k=2, v=3, x=4, u=5, s=6, o=7, fn="rwkv6_wkv_step",
         **mis):
    a = {n: (addr(i, mis.get(n, 0)) if i is not None else None)
         for n, i in dict(r=r, k=k, v=v, x=x, u=u, s=s, o=o).items()}
    return getattr(L, fn)(B, T, H, N, a["r"], a["k"], a["v"], a["x"], a["u"], a["s"],
                          a["o"], None)


def rwkv4_step(L, B=2, T=1, H=1, N=16, k=1, v=2, w=3, u=4, s=5, y=6, **mis):
    a = {n: (addr(i, mis.get(n, 0)) if i is not None else None)
         for n, i in dict(k=k, v=v, w=w, u=u, s=s, y=y).items()}
    return L.rwkv4_wkv_step(B, T, H, N, a["k"], a["v"], a["w"], a["u"], a["s"], a["y"], None)


@pytest.mark.parametrize("dims", [(0, 8, 1, 16), (2, -1, 1, 16), (2, 8, 0, 16),
                                  (2, 8, 1, 0), (1 << 20, 1 << 20, 1, 1 << 10)])
def test_rwkv4_bad_dims(L, dims):
    B, T, H, N = dims
    assert rwkv4(L, B=B, T=T, H=H, N=N) == E_DIM


def test_rwkv4_too_many_channels(L):
    assert rwkv4(L, B=1, T=1, H=1, N=(1 << 20) + 4) == E_UNSUP


@pytest.mark.parametrize("missing", ["k", "v", "w", "u", "y"])
def test_rwkv4_null(L, missing):
    assert rwkv4(L, **{missing: None}) == E_NULL


@pytest.mark.parametrize("which", ["k", "y", "si"])
def test_rwkv4_misaligned(L, which):
    kw = {"k": 1, "v": 2, "w": 3, "u": 4, "si": 5, "so": 6, "y": 7}
    a = {n: addr(i, 2 if n == which else 0) for n, i in kw.items()}
    st = L.rwkv4_wkv_fwd(2, 8, 1, 16, a["k"], a["v"], a["w"], a["u"], a["si"], a["so"],
                         a["y"], None, 0, None)
    assert st == E_ALIGN


def test_rwkv4_output_overlaps_input(L):
    assert rwkv4(L, y=1) == E_ALIAS          # y == k
    assert rwkv4(L, so=3) == E_ALIAS         # state_out == w


def test_rwkv4_outputs_overlap_each_other(L):
    assert rwkv4(L, so=7) == E_ALIAS         # state_out == y


def test_rwkv4_state_partial_overlap(L):
    kw = {"k": 1, "v": 2, "w": 3, "u": 4}
    a = {n: addr(i) for n, i in kw.items()}
    si = ctypes.c_void_p(BASE + 5 * SPAN)
    so = ctypes.c_void_p(BASE + 5 * SPAN + 4)  # overlaps but is not equal
    assert L.rwkv4_wkv_fwd(2, 8, 1, 16, a["k"], a["v"], a["w"], a["u"], si, so,
                           addr(7), None, 0, None) == E_ALIAS


@pytest.mark.parametrize("fn", ["rwkv5_wkv_fwd", "rwkv6_wkv_fwd"])
def test_matrix_head_size_must_be_64(L, fn):
    assert matrix(L, fn, N=32) == E_UNSUP
    assert matrix(L, fn, N=128) == E_UNSUP


@pytest.mark.parametrize("fn", ["rwkv5_wkv_fwd", "rwkv6_wkv_fwd"])
def test_matrix_head_count_limit(L, fn):
    # chunk rows are addressed with 32-bit byte offsets: at most 65536 heads
    assert matrix(L, fn, B=1, T=1, H=65537, si=None, so=None) == E_UNSUP


@pytest.mark.parametrize("fn", ["rwkv5_wkv_fwd", "rwkv6_wkv_fwd"])
@pytest.mark.parametrize("dims", [(0, 8, 2), (2, -3, 2), (2, 8, 0)])
def test_matrix_bad_dims(L, fn, dims):
    B, T, H = dims
    assert matrix(L, fn, B=B, T=T, H=H) == E_DIM


@pytest.mark.parametrize("fn", ["rwkv5_wkv_fwd", "rwkv6_wkv_fwd"])
@pytest.mark.parametrize("missing", ["r", "k", "v", "x", "u", "o"])
def test_matrix_null(L, fn, missing):
    assert matrix(L, fn, **{missing: None}) == E_NULL


@pytest.mark.parametrize("fn", ["rwkv5_wkv_fwd", "rwkv6_wkv_fwd"])
@pytest.mark.parametrize("which", ["r", "x", "si", "so", "o"])
def test_matrix_misaligned(L, fn, which):
    kw = {"r": 1, "k": 2, "v": 3, "x": 4, "u": 5, "si": 6, "so": 7, "o": 8}
    a = {n: addr(i, 8 if n == which else 0) for n, i in kw.items()}
    st = getattr(L, fn)(2, 8, 2, 64, a["r"], a["k"], a["v"], a["x"], a["u"], a["si"],
                        a["so"], a["o"], None, 0, None)
    assert st == E_ALIGN


@pytest.mark.parametrize("fn", ["rwkv5_wkv_fwd", "rwkv6_wkv_fwd"])
def test_matrix_aliasing(L, fn):
    assert matrix(L, fn, o=1) == E_ALIAS    # o == r
    assert matrix(L, fn, o=4) == E_ALIAS    # o == x
    assert matrix(L, fn, so=8) == E_ALIAS   # state_out == o


# ---------------------------------------------------------------------------
# caller workspaces of the forwards

def test_rwkv4_workspace_size(L):
    # none for a single 256-token pass; else the 16 KiB control block and
    # 1.5 KiB of records (6 x 32 channels x 8 bytes) per workgroup:
    # B x ceil(C / 32) channel blocks x ceil(T / 256) passes
    assert L.rwkv4_wkv_fwd_workspace_bytes(8, 256, 1, 768) == 0
    assert L.rwkv4_wkv_fwd_workspace_bytes(8, 1024, 1, 768) == 16384 + 8 * 24 * 4 * 1536
    assert L.rwkv4_wkv_fwd_workspace_bytes(2, 300, 1, 40) == 16384 + 2 * 2 * 2 * 1536
    assert L.rwkv4_wkv_fwd_workspace_bytes(0, 300, 1, 40) == 0


def test_rwkv4_workspace_checks(L):
    need = L.rwkv4_wkv_fwd_workspace_bytes(2, 300, 1, 16)
    assert need > 0
    assert rwkv4(L, T=300, ws=None) == E_NULL
    assert rwkv4(L, T=300, ws_bytes=need - 1) == E_DIM
    assert rwkv4(L, T=300, ws=1) == E_ALIAS      # workspace on k
    assert rwkv4(L, T=300, ws=7) == E_ALIAS      # workspace on y


def test_rwkv4_workspace_misaligned(L):
    a = [addr(i) for i in range(1, 8)]
    need = L.rwkv4_wkv_fwd_workspace_bytes(2, 300, 1, 16)
    assert L.rwkv4_wkv_fwd(2, 300, 1, 16, *a, addr(8, 4), need, None) == E_ALIGN


@pytest.mark.parametrize("fn", ["rwkv5_wkv_fwd", "rwkv6_wkv_fwd"])
def test_matrix_workspace(L, fn):
    # none while every head has a compute unit; with more heads than units
    # (T >= 256) the balanced split's hand-off area
    assert L.rwkv_wkv_fwd_workspace_bytes(2, 8, 2, 64) == 0
    assert L.rwkv_wkv_fwd_workspace_bytes(1, 4096, 200, 64) == 0
    need = L.rwkv_wkv_fwd_workspace_bytes(1, 300, 300, 64)
    assert need > 32768
    assert L.rwkv_wkv_fwd_workspace_bytes(1, 300, 300, 32) == 0
    assert matrix(L, fn, B=1, T=300, H=300, ws=None) == E_NULL
    assert matrix(L, fn, B=1, T=300, H=300, ws_bytes=need - 1) == E_DIM
    a = [addr(i) for i in range(1, 9)]
    assert getattr(L, fn)(1, 300, 300, 64, *a, addr(9, 8), need, None) == E_ALIGN
    assert matrix(L, fn, B=1, T=300, H=300, ws=1) == E_ALIAS   # on r
    assert matrix(L, fn, B=1, T=300, H=300, ws=8) == E_ALIAS   # on o
    assert matrix(L, fn, B=1, T=300, H=300, ws=7) == E_ALIAS   # on state_out


def test_workspace_status_checks(L):
    assert L.rwkv_wkv_workspace_status(None, 1 << 20, None) == E_NULL
    assert L.rwkv_wkv_workspace_status(addr(1), 4096, None) == E_DIM
    assert L.rwkv_wkv_workspace_status(addr(1, 8), 1 << 20, None) == E_ALIGN


STEPS = ["rwkv5_wkv_step", "rwkv6_wkv_step"]


@pytest.mark.parametrize("fn", STEPS)
def test_step_requires_state(L, fn):
    assert step(L, s=None, fn=fn) == E_NULL


@pytest.mark.parametrize("fn", STEPS)
def test_step_rejects_output_on_state(L, fn):
    assert step(L, o=6, fn=fn) == E_ALIAS


@pytest.mark.parametrize("fn", STEPS)
def test_step_head_size(L, fn):
    assert step(L, N=16, fn=fn) == E_UNSUP


@pytest.mark.parametrize("fn", STEPS)
@pytest.mark.parametrize("missing", ["r", "k", "v", "x", "u", "o"])
def test_step_null(L, fn, missing):
    assert step(L, fn=fn, **{missing: None}) == E_NULL


def test_rwkv4_step_requires_state(L):
    assert rwkv4_step(L, s=None) == E_NULL


@pytest.mark.parametrize("missing", ["k", "v", "w", "u", "y"])
def test_rwkv4_step_null(L, missing):
    assert rwkv4_step(L, **{missing: None}) == E_NULL


@pytest.mark.parametrize("dims", [(0, 1, 1, 16), (2, -1, 1, 16), (2, 1, 0, 16)])
def test_rwkv4_step_bad_dims(L, dims):
    B, T, H, N = dims
    assert rwkv4_step(L, B=B, T=T, H=H, N=N) == E_DIM


def test_rwkv4_step_aliasing(L):
    assert rwkv4_step(L, y=5) == E_ALIAS   # y on the state
    assert rwkv4_step(L, s=1) == E_ALIAS   # state on k
    assert rwkv4_step(L, y=2) == E_ALIAS   # y on v


@pytest.mark.parametrize("which", ["k", "s", "y"])
def test_rwkv4_step_misaligned(L, which):
    kw = dict(k=1, v=2, w=3, u=4, s=5, y=6)
    a = {n: addr(i, 2 if n == which else 0) for n, i in kw.items()}
    st = L.rwkv4_wkv_step(2, 1, 1, 16, a["k"], a["v"], a["w"], a["u"], a["s"], a["y"], None)
    assert st == E_ALIGN


def test_rwkv4_step_size_limit(L):
    # one thread per (sequence, channel): B * C up to 2^38
    # (the state, 3 * B * C floats, stays within the per-tensor element limit)
    assert rwkv4_step(L, B=1 << 20, T=1, H=286102, N=1) == E_UNSUP


# ---------------------------------------------------------------------------
# backward

BWD_NAMES = ("r", "k", "v", "x", "u", "si", "do", "dso", "dr", "dk", "dv", "dx", "du", "dsi",
             "ws")


def bwd(L, fn="rwkv6_wkv_bwd", B=2, T=8, H=2, N=64, ws_bytes=None, **over):
    idx = {n: i + 1 for i, n in enumerate(BWD_NAMES)}
    idx.update({n: v for n, v in over.items() if n in idx})
    mis = over.get("mis", {})
    a = {n: (addr(i, mis.get(n, 0)) if i is not None else None) for n, i in idx.items()}
    if ws_bytes is None:
        ws_bytes = L.rwkv_wkv_bwd_workspace_bytes(B, max(T, 1), H, N) if N == 64 else 1 << 20
    return getattr(L, fn)(B, T, H, N, *(a[n] for n in BWD_NAMES[:-1]), a["ws"], ws_bytes, None)


BWDS = ["rwkv5_wkv_bwd", "rwkv6_wkv_bwd"]


def test_bwd_workspace_size(L):
    # the 16 KiB control block, the state entering each 64-token chunk plus
    # the final state, per head, and two per-head partial sums (no hand-off
    # area beyond the control block while every head has a compute unit)
    assert L.rwkv_wkv_bwd_workspace_bytes(2, 130, 3, 64) == \
        16384 + 2 * 3 * 4 * 64 * 64 * 4 + 2 * 2 * 3 * 64 * 4
    assert L.rwkv_wkv_bwd_workspace_bytes(2, 130, 3, 32) == 0
    # with the splits, the hand-off area comes first (256-byte aligned)
    states = 1 * 300 * 6 * 64 * 64 * 4 + 2 * 300 * 64 * 4
    total = L.rwkv_wkv_bwd_workspace_bytes(1, 300, 300, 64)
    assert total > states + 32768 and (total - states) % 256 == 0


@pytest.mark.parametrize("fn", BWDS)
@pytest.mark.parametrize("missing", ["r", "k", "v", "x", "u", "do", "dr", "dk", "dv", "dx", "du",
                                     "ws"])
def test_bwd_null(L, fn, missing):
    assert bwd(L, fn, **{missing: None}) == E_NULL


@pytest.mark.parametrize("fn", BWDS)
def test_bwd_optional_pointers(L, fn):
    # state_in, d_state_out and d_state_in may be NULL; validation then passes
    # and only the launch (on fake addresses) is left, which these tests skip
    # by asking for a too-small workspace
    assert bwd(L, fn, si=None, dso=None, dsi=None, ws_bytes=16) == E_DIM


@pytest.mark.parametrize("fn", BWDS)
def test_bwd_small_workspace(L, fn):
    need = L.rwkv_wkv_bwd_workspace_bytes(2, 8, 2, 64)
    assert bwd(L, fn, ws_bytes=need - 1) == E_DIM


@pytest.mark.parametrize("fn", BWDS)
def test_bwd_head_size_and_dims(L, fn):
    assert bwd(L, fn, N=32) == E_UNSUP
    assert bwd(L, fn, B=0) == E_DIM
    assert bwd(L, fn, T=-1) == E_DIM


@pytest.mark.parametrize("fn", BWDS)
@pytest.mark.parametrize("which", ["r", "do", "dx", "ws", "dsi"])
def test_bwd_misaligned(L, fn, which):
    assert bwd(L, fn, mis={which: 8}) == E_ALIGN


@pytest.mark.parametrize("fn", BWDS)
def test_bwd_aliasing(L, fn):
    assert bwd(L, fn, dr=1) == E_ALIAS    # d_r on r
    assert bwd(L, fn, dx=9) == E_ALIAS    # d_x on d_r
    assert bwd(L, fn, ws=7) == E_ALIAS    # workspace on d_o
    assert bwd(L, fn, mis={"dsi": 16}, dsi=8) == E_ALIAS  # d_state_in partly on d_state_out


# ---------------------------------------------------------------------------
# forward with the output epilogue

def gated(L, fn="rwkv6_wkv_fwd_gated", B=2, T=8, H=2, N=64, eps=1e-5, **over):
    names = ("r", "k", "v", "x", "u", "si", "so", "g", "w", "b", "y")
    idx = {n: i + 1 for i, n in enumerate(names)}
    idx.update({n: val for n, val in over.items() if n in idx})
    mis = over.get("mis", {})
    a = {n: (addr(i, mis.get(n, 0)) if i is not None else None) for n, i in idx.items()}
    return getattr(L, fn)(B, T, H, N, *(a[n] for n in names[:10]), eps, a["y"], None, 0, None)


GATED = ["rwkv5_wkv_fwd_gated", "rwkv6_wkv_fwd_gated"]


@pytest.mark.parametrize("fn", GATED)
@pytest.mark.parametrize("missing", ["r", "x", "u", "g", "w", "b", "y"])
def test_gated_null(L, fn, missing):
    assert gated(L, fn, **{missing: None}) == E_NULL


@pytest.mark.parametrize("fn", GATED)
def test_gated_checks(L, fn):
    assert gated(L, fn, N=32) == E_UNSUP
    assert gated(L, fn, eps=-1.0) == E_DIM
    assert gated(L, fn, eps=float("nan")) == E_DIM
    assert gated(L, fn, mis={"g": 8}) == E_ALIGN
    assert gated(L, fn, y=8) == E_ALIAS   # y on the gate
    assert gated(L, fn, y=1) == E_ALIAS   # y on r


# ---------------------------------------------------------------------------
# Finch decay producer and the forward it feeds

LORA_NAMES = ("x", "sh", "mu", "lam", "a1", "b1", "om", "a2", "b2")


def decay(L, B=2, T=8, D=128, act=1, **over):
    names = LORA_NAMES + ("d",)
    idx = {n: i + 1 for i, n in enumerate(names)}
    idx.update({n: val for n, val in over.items() if n in idx})
    mis = over.get("mis", {})
    a = {n: (addr(i, mis.get(n, 0)) if i is not None else None) for n, i in idx.items()}
    ws = over.get("ws", 12)
    nb = over.get("ws_bytes", L.rwkv6_decay_lora_workspace_bytes(B, T, D))
    return L.rwkv6_decay_lora(B, T, D, act, *(a[n] for n in names),
                              None if ws is None else addr(ws), nb, None)


def fused(L, B=2, T=8, H=2, N=64, act=1, **over):
    names = ("r", "k", "v") + LORA_NAMES + ("u", "si", "so", "o")
    idx = {n: i + 1 for i, n in enumerate(names)}
    idx.update({n: val for n, val in over.items() if n in idx})
    mis = over.get("mis", {})
    a = {n: (addr(i, mis.get(n, 0)) if i is not None else None) for n, i in idx.items()}
    first = [a[n] for n in ("r", "k", "v") + LORA_NAMES]
    ws = over.get("ws", 20)
    nb = over.get("ws_bytes", L.rwkv6_wkv_fwd_lora_workspace_bytes(B, T, H, N))
    return L.rwkv6_wkv_fwd_lora(B, T, H, N, *first, act, a["u"], a["si"], a["so"], a["o"],
                                None if ws is None else addr(ws), nb, None)


@pytest.mark.parametrize("missing", ["x", "mu", "lam", "a1", "b1", "om", "a2", "b2", "d"])
def test_decay_lora_null(L, missing):
    assert decay(L, **{missing: None}) == E_NULL


def test_decay_lora_checks(L):
    assert decay(L, D=96) == E_UNSUP          # D not a multiple of 64
    assert decay(L, B=1, T=1, D=64 * 65536) == E_UNSUP  # more than 65535 channel blocks
    assert decay(L, act=2) == E_DIM
    assert decay(L, B=0) == E_DIM
    assert decay(L, T=-1) == E_DIM
    assert decay(L, B=1 << 16, T=1 << 15) == E_UNSUP  # B T >= 2^31 rows
    assert decay(L, mis={"a2": 8}) == E_ALIGN
    assert decay(L, mis={"sh": 4}) == E_ALIGN
    assert decay(L, d=1) == E_ALIAS           # d on x
    assert decay(L, d=9) == E_ALIAS           # d on B2
    assert decay(L, T=0, d=None) == OK        # nothing to do
    assert decay(L, sh=None, T=0) == OK


def test_decay_lora_workspace(L):
    # act(z A2) of every token (128 bytes, rounded to 256), then the weights
    # laid out as product operands: 16 KiB per block of 64 channels (none
    # past 40 blocks, where the producer streams the block input twice)
    assert L.rwkv6_decay_lora_workspace_bytes(2, 8, 128) == 2 * 8 * 128 + 2 * 16384
    assert L.rwkv6_decay_lora_workspace_bytes(2, 8, 2560) == 2 * 8 * 128 + 40 * 16384
    assert L.rwkv6_decay_lora_workspace_bytes(2, 8, 2624) == 2 * 8 * 128
    assert L.rwkv6_decay_lora_workspace_bytes(2, 8, 96) == 0
    assert decay(L, ws=None) == E_NULL
    assert decay(L, ws_bytes=2 * 8 * 128 + 2 * 16384 - 1) == E_DIM
    assert decay(L, ws=1) == E_ALIAS          # on x
    assert decay(L, ws=10) == E_ALIAS         # on d


def test_fused_workspace(L):
    # the producer's factor (B T 128 bytes) and packed weights after the
    # chunked forward's hand-off area (here only its 16 KiB control block)
    assert L.rwkv6_wkv_fwd_lora_workspace_bytes(2, 8, 2, 64) == 16384 + 2 * 8 * 128 + 2 * 16384
    assert fused(L, ws=None) == E_NULL
    assert fused(L, ws_bytes=100) == E_DIM
    assert fused(L, ws=1) == E_ALIAS          # on r
    assert fused(L, ws=16) == E_ALIAS         # on state_out


@pytest.mark.parametrize("missing", ["r", "x", "a1", "b2", "om", "u", "o"])
def test_fused_null(L, missing):
    assert fused(L, **{missing: None}) == E_NULL


def test_fused_checks(L):
    assert fused(L, N=32) == E_UNSUP
    assert fused(L, act=-1) == E_DIM
    assert fused(L, B=1, T=1, H=65537, si=None, so=None) == E_UNSUP
    assert fused(L, mis={"b1": 8}) == E_ALIGN
    assert fused(L, o=4) == E_ALIAS           # o on the block input
    assert fused(L, so=11) == E_ALIAS         # state_out on B2
    assert fused(L, o=1) == E_ALIAS           # o on r


# ---------------------------------------------------------------------------
# the training pair: a forward that saves the states, a backward that uses them

def fwd_save(L, fn="rwkv6_wkv_fwd_save", B=2, T=8, H=2, N=64, ws_bytes=None, **over):
    names = ("r", "k", "v", "x", "u", "si", "so", "o", "ws")
    idx = {n: i + 1 for i, n in enumerate(names)}
    idx.update({n: val for n, val in over.items() if n in idx})
    mis = over.get("mis", {})
    a = {n: (addr(i, mis.get(n, 0)) if i is not None else None) for n, i in idx.items()}
    if ws_bytes is None:
        ws_bytes = L.rwkv_wkv_bwd_workspace_bytes(B, max(T, 1), H, N)
    return getattr(L, fn)(B, T, H, N, *(a[n] for n in names), ws_bytes, None)


SAVES = ["rwkv5_wkv_fwd_save", "rwkv6_wkv_fwd_save"]


@pytest.mark.parametrize("fn", SAVES)
def test_fwd_save_checks(L, fn):
    need = L.rwkv_wkv_bwd_workspace_bytes(2, 8, 2, 64)
    assert fwd_save(L, fn, ws=None) == E_NULL
    assert fwd_save(L, fn, ws_bytes=need - 1) == E_DIM
    assert fwd_save(L, fn, mis={"ws": 8}) == E_ALIGN
    assert fwd_save(L, fn, ws=1) == E_ALIAS    # workspace on r
    assert fwd_save(L, fn, ws=8) == E_ALIAS    # workspace on o
    assert fwd_save(L, fn, N=32) == E_UNSUP
    assert fwd_save(L, fn, o=None) == E_NULL


@pytest.mark.parametrize("fn", ["rwkv5_wkv_bwd_saved", "rwkv6_wkv_bwd_saved"])
def test_bwd_saved_checks(L, fn):
    names = ("r", "k", "v", "x", "u", "do", "dso", "dr", "dk", "dv", "dx", "du", "dsi", "ws")
    def call(ws_bytes=None, **over):
        idx = {n: i + 1 for i, n in enumerate(names)}
        idx.update(over)
        a = {n: (addr(i) if i is not None else None) for n, i in idx.items()}
        nb = L.rwkv_wkv_bwd_workspace_bytes(2, 8, 2, 64) if ws_bytes is None else ws_bytes
        return getattr(L, fn)(2, 8, 2, 64, *(a[n] for n in names), nb, None)
    assert call(ws=None) == E_NULL
    assert call(ws_bytes=16) == E_DIM
    assert call(dr=1) == E_ALIAS
    assert call(do=None) == E_NULL


# ---------------------------------------------------------------------------
# the allocation-free Finch forward

def noalloc(L, B=2, T=8, H=2, N=64, **over):
    names = ("r", "k", "v", "x", "u", "si", "so", "o")
    idx = {n: i + 1 for i, n in enumerate(names)}
    idx.update({n: val for n, val in over.items() if n in idx})
    a = {n: (addr(i) if i is not None else None) for n, i in idx.items()}
    return L.rwkv6_wkv_fwd_noalloc(B, T, H, N, *(a[n] for n in names), None)


def test_noalloc_checks(L):
    assert noalloc(L, N=32) == E_UNSUP
    assert noalloc(L, B=0) == E_DIM
    assert noalloc(L, r=None) == E_NULL
    assert noalloc(L, o=1) == E_ALIAS
    # a hand-off area beyond its fixed 8 MiB scratch: 600 heads (the four-wave
    # split and its parked states) on 256 compute units
    assert L.rwkv_wkv_fwd_workspace_bytes(2, 320, 300, 64) > 8 << 20
    assert noalloc(L, B=2, T=320, H=300) == E_UNSUP
