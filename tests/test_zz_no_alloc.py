"""The allocation-free Finch forward (rwkv6_wkv_fwd_noalloc), called through
the C ABI, against rwkv6_wkv_fwd with a caller workspace: the same kernels,
so the same bits.  Two calls in a row, the second on a smaller input (the
fixed scratch keeps the first call's contents), and a shape whose hand-off
area exceeds the fixed scratch, which is rejected."""
import ctypes

import pytest

import wkv_synth as S
from helpers import matrix_inputs_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import linear_attention_rnn_wkv_amd as W  # noqa: E402

E_UNSUP = -3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    W.lib()


def noalloc(g, o, so):
    B, T, H, N = g["r"].shape
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return W.lib().rwkv6_wkv_fwd_noalloc(B, T, H, N, p(g["r"]), p(g["k"]), p(g["v"]),
                                         p(g["x"]), p(g["u"]), p(g["s0"]), p(so), p(o), stream)


# 300 heads, 600 tokens: the balanced split in five segments; then 270 heads,
# 320 tokens: sixteen segments (a smaller input); then two heads (no split)
@pytest.mark.parametrize("shapes", [[(1, 600, 300), (2, 320, 135), (1, 100, 2)]])
def test_noalloc_matches_workspace_entry_point(shapes):
    for i, (B, T, H) in enumerate(shapes):
        print(f"noalloc call {i}: B={B} T={T} H={H}", flush=True)
        need = W.fwd_workspace_bytes(B, T, H)
        assert (need > 0) == (i < 2) and need <= 8 << 20
        g = matrix_inputs_dev(S.wkv_inputs(B, T, H, 64, 1300 + i, True, 0.1))
        o = torch.empty_like(g["r"])
        so = torch.empty_like(g["s0"])
        assert noalloc(g, o, so) == 0
        ws = W.new_workspace(need)
        o_ref, s_ref = W.rwkv6_wkv_fwd(g["r"], g["k"], g["v"], g["x"], g["u"], state_in=g["s0"],
                                       workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(so, s_ref)
        assert torch.isfinite(o.float()).all()


def test_noalloc_rejects_a_hand_off_area_beyond_its_scratch():
    B, T, H = 2, 320, 300  # 600 heads: the four-wave split needs about 14 MB
    assert W.fwd_workspace_bytes(B, T, H) > 8 << 20
    g = matrix_inputs_dev(S.wkv_inputs(B, T, H, 64, 1310, True, 0.1))
    o = torch.zeros_like(g["r"])
    so = torch.zeros_like(g["s0"])
    assert noalloc(g, o, so) == E_UNSUP
    torch.cuda.synchronize()
    assert not o.float().any() and not so.any()  # nothing was launched
