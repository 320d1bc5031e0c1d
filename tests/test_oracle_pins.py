"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each check follows from the definitions on the pages (RWKV paper summary,
section "Temporal structure for sequential data processing": decay e^{-w},
bonus e^{u}; RWKV-5/6 summary, sections 4.1.2 "Eagle time mixing" and 4.2.2
"Finch time mixing": matrix state decayed per key channel, bonus u on the
current token, r as the query) or from plain mathematics: explicit sums
evaluated by brute force, geometric series, the w = 1 and w = 0 limits,
hand-worked examples, exact scaling, and split / handoff invariance.
"""
import math

import numpy as np
import pytest

import oracle
import wkv_synth as S
from conftest import read_golden


# ---------------------------------------------------------------------------
# independent brute-force forms

def rwkv4_explicit(k, v, w, u):
    """y_t = sum_{i<=t} a_{t,i} v_i / sum_{i<=t} a_{t,i} with
    a_{t,i} = exp(-(t-1-i) w + k_i) for i < t and exp(u + k_t) for i = t."""
    k = k.astype(np.float64)
    v = v.astype(np.float64)
    w = w.astype(np.float64)
    u = u.astype(np.float64)
    B, T, C = k.shape
    y = np.empty((B, T, C))
    for t in range(T):
        i = np.arange(t)
        expo = -(t - 1 - i)[None, :, None] * w[None, None, :] + k[:, :t, :]
        a = np.exp(expo)
        cur = np.exp(u[None, :] + k[:, t, :])
        y[:, t, :] = (np.sum(a * v[:, :t, :], axis=1) + cur * v[:, t, :]) / (
            np.sum(a, axis=1) + cur)
    return y


def matrix_explicit(r, k, v, x, u, s0):
    """Unrolled Eagle/Finch: with P_i(a, b) = prod_{m=a..b} w_m[i],
    o_t = r_t diag(P(1,t-1)) S_0
        + sum_{s<t} (sum_i r_t[i] P_i(s+1, t-1) k_s[i]) v_s
        + (sum_i r_t[i] u[i] k_t[i]) v_t,
    S_T = diag(P(1,T)) S_0 + sum_{s<=T} diag(P(s+1,T)) k_s^T v_s.
    Products are taken directly, one factor at a time."""
    r, k, v, u, s0 = (a.astype(np.float64) for a in (r, k, v, u, s0))
    B, T, H, N = r.shape
    if x.shape == (H, N):
        w = np.broadcast_to(np.exp(-np.exp(x.astype(np.float64))), (B, T, H, N))
    else:
        w = np.exp(-np.exp(x.astype(np.float64)))

    def P(b, h, a, c):  # 1-indexed inclusive product of decays, per channel
        out = np.ones(N)
        for m in range(a, c + 1):
            out = out * w[b, m - 1, h]
        return out

    o = np.zeros((B, T, H, N))
    sT = np.zeros((B, H, N, N))
    for b in range(B):
        for h in range(H):
            for t in range(1, T + 1):
                rt = r[b, t - 1, h]
                acc = (rt * P(b, h, 1, t - 1)) @ s0[b, h]
                for s in range(1, t):
                    coef = np.sum(rt * P(b, h, s + 1, t - 1) * k[b, s - 1, h])
                    acc = acc + coef * v[b, s - 1, h]
                acc = acc + np.sum(rt * u[h] * k[b, t - 1, h]) * v[b, t - 1, h]
                o[b, t - 1, h] = acc
            st = P(b, h, 1, T)[:, None] * s0[b, h]
            for s in range(1, T + 1):
                st = st + np.outer(P(b, h, s + 1, T) * k[b, s - 1, h], v[b, s - 1, h])
            sT[b, h] = st
    return o, sT


def small_matrix_case(B, T, H, N, seed, per_token=True, s0_sigma=0.3):
    d = S.wkv_inputs(B, T, H, N, seed, per_token, s0_sigma, rkv_sigma=0.5)
    return (S.bf16_to_f32(d["r"]), S.bf16_to_f32(d["k"]), S.bf16_to_f32(d["v"]),
            d["x"], d["u"], d["s0"])


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------------------
# RWKV-4

def test_rwkv4_bruteforce_workload1(oracle_lib):
    d = S.workload(1)
    out = oracle.rwkv4_fwd(d["k"], d["v"], d["w"], d["u"], lib=oracle_lib)
    ref = rwkv4_explicit(d["k"], d["v"], d["w"], d["u"])
    assert np.max(np.abs(out["y"] - ref) / np.maximum(np.abs(ref), out["scale"])) < 1e-12


def test_rwkv4_bruteforce_with_history(oracle_lib):
    # a history of P tokens given as (num, den) must equal running them inline
    d = S.rwkv4_inputs(2, 40, 5, 11, k_sigma=2.0)
    P = 17
    head = oracle.rwkv4_fwd(d["k"][:, :P], d["v"][:, :P], d["w"], d["u"], lib=oracle_lib)
    tail = oracle.rwkv4_fwd(d["k"][:, P:], d["v"][:, P:], d["w"], d["u"],
                            head["num"], head["den"], lib=oracle_lib)
    ref = rwkv4_explicit(d["k"], d["v"], d["w"], d["u"])
    assert rel(tail["y"], ref[:, P:]) < 1e-12
    assert rel(head["y"], ref[:, :P]) < 1e-12


def test_rwkv4_constant_inputs_closed_form(oracle_lib):
    # constant k and v: every weighted average equals v; the denominator is a
    # geometric series: Den_T = e^k (1 - e^{-T w}) / (1 - e^{-w})
    B, T, C = 1, 50, 4
    k = np.full((B, T, C), 0.75, np.float32)
    v = np.full((B, T, C), -1.25, np.float32)
    w = np.array([0.01, 0.3, 1.0, 4.0], np.float32)
    u = np.array([0.5, -0.5, 2.0, 0.0], np.float32)
    out = oracle.rwkv4_fwd(k, v, w, u, lib=oracle_lib)
    np.testing.assert_allclose(out["y"], -1.25, rtol=1e-14)
    wd = w.astype(np.float64)
    den = math.exp(0.75) * (1 - np.exp(-T * wd)) / (1 - np.exp(-wd))
    np.testing.assert_allclose(out["den"][0], den, rtol=1e-13)
    np.testing.assert_allclose(out["num"][0], -1.25 * den, rtol=1e-13)


def test_rwkv4_first_token_is_v(oracle_lib):
    d = S.rwkv4_inputs(3, 4, 16, 12, k_sigma=3.0)
    out = oracle.rwkv4_fwd(d["k"], d["v"], d["w"], d["u"], lib=oracle_lib)
    np.testing.assert_allclose(out["y"][:, 0], d["v"][:, 0].astype(np.float64), rtol=1e-15)


def test_rwkv4_golden_hand_example(oracle_lib):
    g = read_golden("rwkv4_hand.txt")
    k = np.array(g["k"], np.float32).reshape(1, 3, 1)
    v = np.array(g["v"], np.float32).reshape(1, 3, 1)
    out = oracle.rwkv4_fwd(k, v, np.array(g["w"], np.float32),
                           np.array(g["u"], np.float32), lib=oracle_lib)
    np.testing.assert_allclose(out["y"].ravel(), g["y"], rtol=1e-6)
    np.testing.assert_allclose(out["num"].ravel(), g["num"], rtol=1e-6)
    np.testing.assert_allclose(out["den"].ravel(), g["den"], rtol=1e-6)


def test_rwkv4_split_invariance_bitwise(oracle_lib):
    d = S.rwkv4_inputs(2, 64, 8, 13)
    full = oracle.rwkv4_fwd(d["k"], d["v"], d["w"], d["u"], lib=oracle_lib)
    a = oracle.rwkv4_fwd(d["k"][:, :23], d["v"][:, :23], d["w"], d["u"], lib=oracle_lib)
    b = oracle.rwkv4_fwd(d["k"][:, 23:], d["v"][:, 23:], d["w"], d["u"],
                         a["num"], a["den"], lib=oracle_lib)
    assert np.array_equal(np.concatenate([a["y"], b["y"]], 1), full["y"])
    assert np.array_equal(b["num"], full["num"]) and np.array_equal(b["den"], full["den"])


def test_rwkv4_is_ratio_of_two_matrix_recurrences(oracle_lib):
    # With N = 1, r = 1, k' = e^k, w' = e^{-w} (x = ln w), u' = e^u the matrix
    # recurrence yields Num_{t-1} + e^{u+k_t} v_t; with v = 1 it yields the
    # denominator.  Their ratio is the RWKV-4 output.
    d = S.rwkv4_inputs(2, 30, 6, 14)
    B, T, C = d["k"].shape
    k4 = np.moveaxis(np.exp(d["k"].astype(np.float64)), 2, 1).reshape(B * C, T, 1, 1)
    v4 = np.moveaxis(d["v"], 2, 1).reshape(B * C, T, 1, 1)
    num = []
    den = []
    for c in range(C):
        sel = slice(c, B * C, C)
        x = np.full((1, 1), math.log(float(d["w"][c])), np.float32)
        uu = np.full((1, 1), math.exp(float(d["u"][c])), np.float32)
        ones = np.ones_like(v4[sel], np.float32)
        o_num, _ = oracle.wkv_matrix(ones, k4[sel], v4[sel], x, uu, lib=oracle_lib)
        o_den, _ = oracle.wkv_matrix(ones, k4[sel], ones, x, uu, lib=oracle_lib)
        num.append(o_num[:, :, 0, 0])
        den.append(o_den[:, :, 0, 0])
    y_mat = np.stack(num, -1) / np.stack(den, -1)
    out = oracle.rwkv4_fwd(d["k"], d["v"], d["w"], d["u"], lib=oracle_lib)
    assert np.max(np.abs(y_mat - out["y"]) / out["scale"]) < 1e-5


# ---------------------------------------------------------------------------
# Eagle / Finch

@pytest.mark.parametrize("per_token", [False, True])
def test_matrix_bruteforce(oracle_lib, per_token):
    r, k, v, x, u, s0 = small_matrix_case(2, 13, 2, 8, 21 + per_token, per_token)
    o, sT = oracle.wkv_matrix(r, k, v, x, u, s0, lib=oracle_lib)
    o_ref, s_ref = matrix_explicit(r, k, v, x, u, s0)
    assert rel(o, o_ref) < 1e-12
    assert rel(sT, s_ref) < 1e-12


def test_matrix_bruteforce_head_size_64(oracle_lib):
    r, k, v, x, u, s0 = small_matrix_case(1, 6, 1, 64, 23, True)
    o, sT = oracle.wkv_matrix(r, k, v, x, u, s0, lib=oracle_lib)
    o_ref, s_ref = matrix_explicit(r, k, v, x, u, s0)
    assert rel(o, o_ref) < 1e-12
    assert rel(sT, s_ref) < 1e-12


def test_matrix_golden_hand_example(oracle_lib):
    g = read_golden("wkv_matrix_hand.txt")
    r = np.array(g["r"], np.float32).reshape(1, 2, 1, 2)
    k = np.array(g["k"], np.float32).reshape(1, 2, 1, 2)
    v = np.array(g["v"], np.float32).reshape(1, 2, 1, 2)
    x = np.array(g["x"], np.float32).reshape(1, 2, 1, 2)
    u = np.array(g["u"], np.float32).reshape(1, 2)
    s0 = np.array(g["s0"]).reshape(1, 1, 2, 2)
    o, s2 = oracle.wkv_matrix(r, k, v, x, u, s0, lib=oracle_lib)
    np.testing.assert_allclose(o.ravel(), g["o"], rtol=1e-6, atol=1e-12)
    np.testing.assert_allclose(s2.ravel(), g["s2"], rtol=1e-6, atol=1e-12)
    _, s1 = oracle.wkv_matrix(r[:, :1], k[:, :1], v[:, :1], x[:, :1], u, s0, lib=oracle_lib)
    np.testing.assert_allclose(s1.ravel(), g["s1"], rtol=1e-6, atol=1e-12)


def test_matrix_geometric_closed_form(oracle_lib):
    # static w, constant k and v:
    #   S_{t-1} = diag(w^{t-1}) S_0 + diag((1 - w^{t-1}) / (1 - w)) k^T v
    B, T, H, N = 1, 40, 1, 4
    rng = np.random.default_rng(5)
    kk = rng.normal(size=N).astype(np.float32)
    vv = rng.normal(size=N).astype(np.float32)
    r = rng.normal(size=(B, T, H, N)).astype(np.float32)
    k = np.broadcast_to(kk, (B, T, H, N)).copy()
    v = np.broadcast_to(vv, (B, T, H, N)).copy()
    x = np.array([[-4.0, -1.5, -0.5, 0.7]], np.float32)
    u = rng.normal(size=(H, N)).astype(np.float32)
    s0 = rng.normal(size=(B, H, N, N))
    o, sT = oracle.wkv_matrix(r, k, v, x, u, s0, lib=oracle_lib)
    w = np.exp(-np.exp(x[0].astype(np.float64)))
    kv = np.outer(kk.astype(np.float64), vv.astype(np.float64))
    for t in range(1, T + 1):
        wt = w ** (t - 1)
        st = wt[:, None] * s0[0, 0] + ((1 - wt) / (1 - w))[:, None] * kv
        rt = r[0, t - 1, 0].astype(np.float64)
        expect = rt @ st + np.sum(rt * u[0] * kk) * vv
        np.testing.assert_allclose(o[0, t - 1, 0], expect, rtol=1e-11, atol=1e-12)
    wt = w ** T
    np.testing.assert_allclose(
        sT[0, 0], wt[:, None] * s0[0, 0] + ((1 - wt) / (1 - w))[:, None] * kv,
        rtol=1e-11, atol=1e-12)


def test_matrix_no_decay_is_causal_linear_attention(oracle_lib):
    # x = -200 gives w = exp(-exp(-200)) = 1 exactly: the WKV becomes causal
    # linear attention with a bonus diagonal:
    #   O = tril(R K^T, -1) V + diag(R diag(u) K^T) V + R S_0
    r, k, v, _, u, s0 = small_matrix_case(1, 24, 1, 16, 31, True)
    x = np.full(r.shape, -200.0, np.float32)
    o, sT = oracle.wkv_matrix(r, k, v, x, u, s0, lib=oracle_lib)
    R, K, V = (a[0, :, 0].astype(np.float64) for a in (r, k, v))
    A = np.tril(R @ K.T, -1)
    bonus = np.einsum("ti,i,ti->t", R, u[0].astype(np.float64), K)
    expect = A @ V + bonus[:, None] * V + R @ s0[0, 0]
    np.testing.assert_allclose(o[0, :, 0], expect, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sT[0, 0], s0[0, 0] + K.T @ V, rtol=1e-12, atol=1e-12)


def test_matrix_full_decay_keeps_only_last_token(oracle_lib):
    # x = +10 gives w = exp(-e^10) = 0: S_t = k_t^T v_t, so
    # o_t = (r_t . k_{t-1}) v_{t-1} + (r_t u . k_t) v_t, and o_1 = r_1 S_0 + bonus.
    r, k, v, _, u, s0 = small_matrix_case(1, 10, 1, 8, 32, True)
    x = np.full(r.shape, 10.0, np.float32)
    o, sT = oracle.wkv_matrix(r, k, v, x, u, s0, lib=oracle_lib)
    R, K, V = (a[0, :, 0].astype(np.float64) for a in (r, k, v))
    uu = u[0].astype(np.float64)
    for t in range(10):
        prev = R[t] @ s0[0, 0] if t == 0 else (R[t] @ K[t - 1]) * V[t - 1]
        expect = prev + np.sum(R[t] * uu * K[t]) * V[t]
        np.testing.assert_allclose(o[0, t, 0], expect, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sT[0, 0], np.outer(K[-1], V[-1]), rtol=1e-15)


def test_matrix_single_token(oracle_lib):
    # T = 1: o = r (S_0 + diag(u) k^T v), S_1 = diag(w) S_0 + k^T v
    r, k, v, x, u, s0 = small_matrix_case(2, 1, 3, 8, 33, True)
    o, s1 = oracle.wkv_matrix(r, k, v, x, u, s0, lib=oracle_lib)
    for b in range(2):
        for h in range(3):
            rr, kk, vv = (a[b, 0, h].astype(np.float64) for a in (r, k, v))
            M = s0[b, h] + np.diag(u[h].astype(np.float64)) @ np.outer(kk, vv)
            np.testing.assert_allclose(o[b, 0, h], rr @ M, rtol=1e-12, atol=1e-14)
            w = np.exp(-np.exp(x[b, 0, h].astype(np.float64)))
            np.testing.assert_allclose(s1[b, h], w[:, None] * s0[b, h] + np.outer(kk, vv),
                                       rtol=1e-13, atol=1e-15)


def test_finch_with_constant_logits_equals_eagle_bitwise(oracle_lib):
    r, k, v, x, u, s0 = small_matrix_case(2, 20, 2, 16, 34, False)
    xt = np.broadcast_to(x, r.shape).copy()
    o_e, s_e = oracle.wkv_matrix(r, k, v, x, u, s0, lib=oracle_lib)
    o_f, s_f = oracle.wkv_matrix(r, k, v, xt, u, s0, lib=oracle_lib)
    assert np.array_equal(o_e, o_f) and np.array_equal(s_e, s_f)


@pytest.mark.parametrize("cut", [1, 17, 31])
def test_matrix_split_invariance_bitwise(oracle_lib, cut):
    r, k, v, x, u, s0 = small_matrix_case(2, 32, 2, 8, 35, True)
    o, sT = oracle.wkv_matrix(r, k, v, x, u, s0, lib=oracle_lib)
    o1, s1 = oracle.wkv_matrix(r[:, :cut], k[:, :cut], v[:, :cut], x[:, :cut], u, s0,
                               lib=oracle_lib)
    o2, s2 = oracle.wkv_matrix(r[:, cut:], k[:, cut:], v[:, cut:], x[:, cut:], u, s1,
                               lib=oracle_lib)
    assert np.array_equal(np.concatenate([o1, o2], 1), o)
    assert np.array_equal(s2, sT)


@pytest.mark.parametrize("per_token", [False, True], ids=["eagle", "finch"])
def test_matrix_stepwise_equals_sequence_bitwise(oracle_lib, per_token):
    # decoding one token per call with the state handed over equals one call
    r, k, v, x, u, s0 = small_matrix_case(1, 12, 2, 8, 36, per_token)
    o, sT = oracle.wkv_matrix(r, k, v, x, u, s0, lib=oracle_lib)
    s = s0.astype(np.float64)
    for t in range(12):
        xt = x[:, t:t + 1] if per_token else x
        ot, s = oracle.wkv_matrix(r[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], xt, u, s,
                                  lib=oracle_lib)
        assert np.array_equal(ot[:, 0], o[:, t])
    assert np.array_equal(s, sT)


def test_rwkv4_stepwise_equals_sequence_bitwise(oracle_lib):
    # RWKV-4 decoding: one token per call, the (Num, Den) history handed over
    d = S.rwkv4_inputs(2, 12, 8, 37, k_sigma=2.0)
    full = oracle.rwkv4_fwd(d["k"], d["v"], d["w"], d["u"], lib=oracle_lib)
    num = den = None
    for t in range(12):
        out = oracle.rwkv4_fwd(d["k"][:, t:t + 1], d["v"][:, t:t + 1], d["w"], d["u"],
                               num, den, lib=oracle_lib)
        assert np.array_equal(out["y"][:, 0], full["y"][:, t])
        num, den = out["num"], out["den"]
    assert np.array_equal(num, full["num"]) and np.array_equal(den, full["den"])


def test_matrix_scaling_exact(oracle_lib):
    # linear in (v, S_0) jointly and in r alone; powers of two scale exactly
    r, k, v, x, u, s0 = small_matrix_case(1, 16, 2, 8, 37, True)
    o, sT = oracle.wkv_matrix(r, k, v, x, u, s0, lib=oracle_lib)
    o2, s2 = oracle.wkv_matrix(r, k, 2 * v, x, u, 2 * s0, lib=oracle_lib)
    assert np.array_equal(o2, 2 * o) and np.array_equal(s2, 2 * sT)
    o4, s4 = oracle.wkv_matrix(4 * r, k, v, x, u, s0, lib=oracle_lib)
    assert np.array_equal(o4, 4 * o) and np.array_equal(s4, sT)


def test_matrix_additive_in_v(oracle_lib):
    r, k, v, x, u, s0 = small_matrix_case(1, 16, 2, 8, 38, True)
    _, _, v2, _, _, s02 = small_matrix_case(1, 16, 2, 8, 39, True)
    oa, sa = oracle.wkv_matrix(r, k, v, x, u, s0, lib=oracle_lib)
    ob, sb = oracle.wkv_matrix(r, k, v2, x, u, s02, lib=oracle_lib)
    vs = v + v2  # exact: sums of two bf16 values of similar size fit in fp32
    assert np.array_equal(vs.astype(np.float64), v.astype(np.float64) + v2.astype(np.float64))
    oc, sc = oracle.wkv_matrix(r, k, vs, x, u, s0.astype(np.float64) + s02, lib=oracle_lib)
    np.testing.assert_allclose(oc, oa + ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sc, sa + sb, rtol=1e-12, atol=1e-13)


def test_matrix_heads_and_batches_are_independent(oracle_lib):
    r, k, v, x, u, s0 = small_matrix_case(2, 9, 3, 8, 40, True)
    o, sT = oracle.wkv_matrix(r, k, v, x, u, s0, lib=oracle_lib)
    for b in range(2):
        for h in range(3):
            ob, sb = oracle.wkv_matrix(r[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1],
                                       v[b:b + 1, :, h:h + 1], x[b:b + 1, :, h:h + 1],
                                       u[h:h + 1], s0[b:b + 1, h:h + 1], lib=oracle_lib)
            assert np.array_equal(ob[0, :, 0], o[b, :, h])
            assert np.array_equal(sb[0, 0], sT[b, h])


def test_thread_count_does_not_change_results(oracle_lib):
    r, k, v, x, u, s0 = small_matrix_case(2, 10, 3, 8, 41, True)
    a = oracle.wkv_matrix(r, k, v, x, u, s0, nthreads=1, lib=oracle_lib)
    b = oracle.wkv_matrix(r, k, v, x, u, s0, nthreads=5, lib=oracle_lib)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# Eagle / Finch backward

def _loss(r, k, v, x, u, s0, G, Hs, lib):
    o, sT = oracle.wkv_matrix(r, k, v, x, u, s0, lib=lib)
    return float(np.sum(o * G) + np.sum(sT * Hs))


def _bwd_case(T, per_token, seed, N=4, H=1, B=1):
    r, k, v, x, u, s0 = small_matrix_case(B, T, H, N, seed, per_token)
    g = np.random.default_rng(seed)
    G = g.standard_normal((B, T, H, N))
    Hs = g.standard_normal((B, H, N, N))
    return r, k, v, x, u, s0, G, Hs


@pytest.mark.parametrize("per_token", [False, True], ids=["eagle", "finch"])
@pytest.mark.parametrize("T", [5, 70])
def test_matrix_bwd_finite_differences(oracle_lib, per_token, T):
    # Every gradient entry against central differences of the forward oracle:
    # the step 2^-12 is exact on these fp32 inputs (|value| < 2^11), so the
    # difference quotient is the fp64 derivative up to O(h^2).  T = 70 crosses
    # the backward's 64-token recomputation segment.
    r, k, v, x, u, s0, G, Hs = _bwd_case(T, per_token, 40 + T)
    got = oracle.wkv_matrix_bwd(r, k, v, x, u, G, s0, Hs, lib=oracle_lib)
    h = 2.0 ** -12
    args = dict(r=r, k=k, v=v, x=x, u=u)
    names = {"r": "dr", "k": "dk", "v": "dv", "x": "dx", "u": "du"}
    for name, a in args.items():
        fd = np.zeros(a.shape)
        for idx in np.ndindex(a.shape):
            lo, hi = (dict(args), dict(args))
            for sgn, dct in ((-1, lo), (1, hi)):
                p = a.copy()
                p[idx] = np.float32(p[idx] + sgn * h)
                assert p[idx] == a[idx] + sgn * h
                dct[name] = p
            fd[idx] = (_loss(hi["r"], hi["k"], hi["v"], hi["x"], hi["u"], s0, G, Hs,
                             oracle_lib) -
                       _loss(lo["r"], lo["k"], lo["v"], lo["x"], lo["u"], s0, G, Hs,
                             oracle_lib)) / (2 * h)
        ref = got[names[name]]
        scale = max(np.max(np.abs(fd)), 1e-12)
        assert np.max(np.abs(ref - fd)) <= 2e-6 * scale, (name, np.max(np.abs(ref - fd)), scale)
    # the initial state (fp64 input): a smaller step, all entries
    fd = np.zeros(s0.shape)
    hs = 1e-6
    for idx in np.ndindex(s0.shape):
        p, m = s0.astype(np.float64), s0.astype(np.float64)
        p[idx] += hs
        m[idx] -= hs
        fd[idx] = (_loss(r, k, v, x, u, p, G, Hs, oracle_lib) -
                   _loss(r, k, v, x, u, m, G, Hs, oracle_lib)) / (2 * hs)
    assert np.max(np.abs(got["ds0"] - fd)) <= 1e-6 * max(np.max(np.abs(fd)), 1e-12)


def test_matrix_bwd_no_decay_is_linear_attention_backward(oracle_lib):
    # x = -200 makes w = 1 in fp64: the forward is causal linear attention
    # O = tril(R K^T, -1) V + diag(R diag(u) K^T) V + R S0, S_T = S0 + K^T V,
    # whose gradients are plain matrix products (numpy)
    T, N = 40, 8
    r, k, v, x, u, s0, G, Hs = _bwd_case(T, True, 77, N=N)
    x = np.full_like(x, -200.0)
    got = oracle.wkv_matrix_bwd(r, k, v, x, u, G, s0, Hs, lib=oracle_lib)
    R, K, V = (a[0, :, 0].astype(np.float64) for a in (r, k, v))
    uu, S0, dO, dST = u[0].astype(np.float64), s0[0, 0], G[0, :, 0], Hs[0, 0]
    dM = dO @ V.T
    dMl = np.tril(dM, -1)
    dd = np.diag(dM)
    beta = np.sum(R * uu * K, axis=1)
    M = np.tril(R @ K.T, -1) + np.diag(beta)
    dR = dMl @ K + (uu * K) * dd[:, None] + dO @ S0.T
    dK = dMl.T @ R + (uu * R) * dd[:, None] + V @ dST.T
    dV = M.T @ dO + K @ dST
    dS0 = R.T @ dO + dST
    du = np.sum(R * K * dd[:, None], axis=0)
    for name, want in (("dr", dR), ("dk", dK), ("dv", dV)):
        assert np.allclose(got[name][0, :, 0], want, rtol=1e-12, atol=1e-12), name
    assert np.allclose(got["ds0"][0, 0], dS0, rtol=1e-12, atol=1e-12)
    assert np.allclose(got["du"][0], du, rtol=1e-12, atol=1e-12)
    assert np.max(np.abs(got["dx"])) < 1e-80  # dw/dx = -w e^x, e^-200 ~ 1e-87


def test_matrix_bwd_eagle_decay_gradient_is_finch_summed(oracle_lib):
    # Eagle's x is Finch's x repeated over sequences and tokens, so its
    # gradient is the sum of Finch's per-token gradients
    B, T, H, N = 2, 30, 2, 8
    r, k, v, x, u, s0, G, Hs = _bwd_case(T, False, 78, N=N, H=H, B=B)
    xf = np.broadcast_to(x, (B, T, H, N)).copy()
    e = oracle.wkv_matrix_bwd(r, k, v, x, u, G, s0, Hs, lib=oracle_lib)
    f = oracle.wkv_matrix_bwd(r, k, v, xf, u, G, s0, Hs, lib=oracle_lib)
    assert np.allclose(e["dx"], f["dx"].sum(axis=(0, 1)), rtol=1e-12, atol=1e-14)
    for n in ("dr", "dk", "dv", "du", "ds0"):
        assert np.array_equal(e[n], f[n]), n


# ---------------------------------------------------------------------------
# output epilogue: LayerNorm per head (GroupNorm over heads), SiLU gate

def _ng_case(seed, rows=6, H=3, N=8):
    g = np.random.default_rng(seed)
    o = g.standard_normal((rows, H, N)) * 3 + 1
    gate = g.standard_normal((rows, H, N)).astype(np.float32)
    w = (g.standard_normal((H, N)) * 0.5 + 1).astype(np.float32)
    b = (g.standard_normal((H, N)) * 0.2).astype(np.float32)
    return o, gate, w, b


def test_norm_gate_is_group_norm_times_silu(oracle_lib):
    # against torch's group_norm (float64, CPU) and silu: one group per head
    torch = pytest.importorskip("torch")
    o, gate, w, b = _ng_case(1)
    rows, H, N = o.shape
    got = oracle.norm_gate(o, gate, w, b, 1e-5, lib=oracle_lib)
    t = torch.from_numpy(o.reshape(rows, H * N))
    gn = torch.nn.functional.group_norm(t, H, torch.from_numpy(w.reshape(-1)).double(),
                                        torch.from_numpy(b.reshape(-1)).double(), eps=1e-5)
    want = gn.numpy().reshape(o.shape) * torch.nn.functional.silu(
        torch.from_numpy(gate).double()).numpy()
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_norm_gate_normalises_each_head(oracle_lib):
    # unit weight, zero bias, a gate large enough that silu(g) = g to fp64:
    # y / g has zero mean and (for eps = 0) unit variance per head and token
    o, gate, w, b = _ng_case(2)
    gate = np.full_like(gate, 40.0)
    y = oracle.norm_gate(o, gate, np.ones_like(w), np.zeros_like(b), 0.0, lib=oracle_lib) / 40.0
    assert np.allclose(y.mean(axis=-1), 0.0, atol=1e-12)
    assert np.allclose((y ** 2).mean(axis=-1), 1.0, rtol=1e-12)


def test_norm_gate_affine_and_gate_structure(oracle_lib):
    o, gate, w, b = _ng_case(3)
    base = oracle.norm_gate(o, np.full_like(gate, 40.0), np.ones_like(w), np.zeros_like(b),
                            1e-3, lib=oracle_lib) / 40.0
    y = oracle.norm_gate(o, gate, w, b, 1e-3, lib=oracle_lib)
    silu = gate / (1.0 + np.exp(-gate.astype(np.float64)))
    assert np.allclose(y, (base * w + b) * silu, rtol=1e-12, atol=1e-13)
    # a zero gate closes the output; shifting o by a constant per head changes nothing
    assert not np.any(oracle.norm_gate(o, np.zeros_like(gate), w, b, 1e-3, lib=oracle_lib))
    shifted = oracle.norm_gate(o + 7.0, gate, w, b, 1e-3, lib=oracle_lib)
    assert np.allclose(shifted, y, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# Finch decay producer: ddlerp and LoRA_omega (RWKV-5/6 summary 4.2.1, 4.2.2)

def _dl_case(seed, B=2, T=7, D=12, R1=3, R2=5):
    g = np.random.default_rng(seed)
    f = lambda *s: g.standard_normal(s).astype(np.float32)
    return dict(x=f(B, T, D), shift=f(B, D), mu_x=g.random(D).astype(np.float32),
                lam=g.random(D).astype(np.float32), A1=f(D, R1) * 0.3, B1=f(R1, D) * 0.3,
                omega=f(D) - 3.0, A2=f(D, R2) * 0.3, B2=f(R2, D) * 0.4)


def _dl(c, lib, act="tanh", **over):
    a = dict(c)
    a.update(over)
    return oracle.decay_lora(a["x"], a["mu_x"], a["lam"], a["A1"], a["B1"], a["omega"],
                             a["A2"], a["B2"], act=act, shift=a["shift"], lib=lib)


def _prev(c):
    # x_{t-1}, with the shift row before the first token
    return np.concatenate([c["shift"][:, None, :], c["x"][:, :-1, :]], axis=1).astype(np.float64)


def test_decay_lora_without_offset_is_omega(oracle_lib):
    # B_omega = 0 (or A_omega = 0 under tanh) leaves the learned logit omega:
    # Eagle's static decay, whatever the input
    c = _dl_case(11)
    for act in ("identity", "tanh"):
        d = _dl(c, oracle_lib, act, B2=np.zeros_like(c["B2"]))
        assert np.array_equal(d, np.broadcast_to(c["omega"].astype(np.float64), d.shape))
    d = _dl(c, oracle_lib, "tanh", A2=np.zeros_like(c["A2"]))
    assert np.array_equal(d, np.broadcast_to(c["omega"].astype(np.float64), d.shape))


def test_decay_lora_constant_sequence(oracle_lib):
    # x_t = x_{t-1} for every t: the interpolation returns x whatever its mix,
    # so d = omega + act(x A2) B2 (numpy products), independent of mu, lam, A1, B1
    c = _dl_case(12)
    row = c["x"][:, :1, :]
    c["x"] = np.repeat(row, c["x"].shape[1], axis=1)
    c["shift"] = row[:, 0, :].copy()
    xr = c["x"].astype(np.float64)
    for act, fn in (("identity", lambda s: s), ("tanh", np.tanh)):
        want = c["omega"].astype(np.float64) + fn(xr @ c["A2"].astype(np.float64)) @ c["B2"].astype(np.float64)
        got = _dl(c, oracle_lib, act)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
        got2 = _dl(c, oracle_lib, act, mu_x=1 - c["mu_x"], lam=c["lam"] * 3, A1=-c["A1"],
                   B1=c["B1"] * 2)
        assert np.allclose(got2, got, rtol=1e-12, atol=1e-12)


def test_decay_lora_full_and_no_shift(oracle_lib):
    # B1 = 0: the mix is lam alone.  lam = 1 takes the previous token (the
    # shift row before the first), lam = 0 the current one; either way the
    # decay is omega + act(. A2) B2 (numpy products)
    c = _dl_case(13)
    A2, B2, om = (c[n].astype(np.float64) for n in ("A2", "B2", "omega"))
    for lam, src in ((1.0, _prev(c)), (0.0, c["x"].astype(np.float64))):
        got = _dl(c, oracle_lib, "tanh", B1=np.zeros_like(c["B1"]),
                  lam=np.full_like(c["lam"], lam))
        assert np.allclose(got, om + np.tanh(src @ A2) @ B2, rtol=1e-12, atol=1e-12)
    # lam = 1/2: the midpoint
    got = _dl(c, oracle_lib, "identity", B1=np.zeros_like(c["B1"]),
              lam=np.full_like(c["lam"], 0.5))
    mid = 0.5 * (_prev(c) + c["x"].astype(np.float64))
    assert np.allclose(got, om + (mid @ A2) @ B2, rtol=1e-12, atol=1e-12)


def test_decay_lora_mix_lora_structure(oracle_lib):
    # A2 = B2 = I, omega = 0, identity: d exposes z = x + dx * m.  The part of
    # z that the mix's LoRA adds, divided by dx, is (y A1) B1 = y (A1 B1) with
    # y = x (mu = 0) or y = x_{t-1} (mu = 1), and it is linear in B1
    c = _dl_case(14, R2=12)
    D = c["x"].shape[-1]
    eye = np.eye(D, dtype=np.float32)
    base = dict(A2=eye, B2=eye, omega=np.zeros(D, np.float32))
    dx = _prev(c) - c["x"].astype(np.float64)
    AB = c["A1"].astype(np.float64) @ c["B1"].astype(np.float64)
    z0 = _dl(c, oracle_lib, "identity", B1=np.zeros_like(c["B1"]), **base)
    for mu, y in ((0.0, c["x"].astype(np.float64)), (1.0, _prev(c))):
        z = _dl(c, oracle_lib, "identity", mu_x=np.full_like(c["mu_x"], mu), **base)
        assert np.allclose((z - z0) / dx, y @ AB, rtol=1e-9, atol=1e-9)
        z2 = _dl(c, oracle_lib, "identity", mu_x=np.full_like(c["mu_x"], mu),
                 B1=c["B1"] * 2, **base)
        assert np.allclose(z2 - z0, 2 * (z - z0), rtol=1e-12, atol=1e-12)


def test_decay_lora_tanh_saturates(oracle_lib):
    # a huge A_omega saturates tanh: d = omega + sign(x A2) B2 (mix lam = 0)
    c = _dl_case(15)
    got = _dl(c, oracle_lib, "tanh", A2=c["A2"] * 1e6, B1=np.zeros_like(c["B1"]),
              lam=np.zeros_like(c["lam"]))
    s = np.sign(c["x"].astype(np.float64) @ c["A2"].astype(np.float64))
    want = c["omega"].astype(np.float64) + s @ c["B2"].astype(np.float64)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_decay_lora_split_and_channel_locality(oracle_lib):
    # a split sequence with the first part's last token as the shift row gives
    # the same bits; channel i of d depends on column i of B2 and omega only
    c = _dl_case(16, T=9)
    full = _dl(c, oracle_lib)
    a = dict(c, x=c["x"][:, :4].copy())
    b = dict(c, x=c["x"][:, 4:].copy(), shift=c["x"][:, 3].copy())
    assert np.array_equal(np.concatenate([_dl(a, oracle_lib), _dl(b, oracle_lib)], axis=1), full)
    B2 = c["B2"].copy()
    B2[:, 5] += 1.0
    om = c["omega"].copy()
    om[7] -= 2.0
    got = _dl(c, oracle_lib, B2=B2, omega=om)
    keep = [i for i in range(full.shape[-1]) if i not in (5, 7)]
    assert np.array_equal(got[..., keep], full[..., keep])
    assert np.allclose(got[..., 7], full[..., 7] - 2.0, rtol=0, atol=1e-12)
    assert not np.allclose(got[..., 5], full[..., 5])
