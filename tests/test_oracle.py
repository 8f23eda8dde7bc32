"""Pins for the CPU oracle (runs without a GPU).

The pages print no worked numeric example for the attention forward pass, so
the oracle is pinned to what the mathematics fixes: closed forms for special
inputs, invariants of the definition, a library special case (torch's fp64
scaled-dot-product attention plus logsumexp, the reference the Triton test
harness of "FlashAttention-2 from PyTorch to Triton" uses) and a 50-digit
brute force on tiny inputs.

Each pin is a ``check_*`` function taking the attention callable, so the same
pins also run against deliberately broken builds of the oracle
(``test_pins_catch_planted_mistakes``): a dropped scale, a wrong log base, an
excluded diagonal, a reversed causal mask, a dropped normalisation or a
misindexed operand must each fail at least one pin.
"""
import decimal
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from workloads import make_inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def rnd(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal(shape) * scale).astype(np.float32)


def close(a, b, atol):
    np.testing.assert_allclose(a, b, rtol=0, atol=atol)


# ---------------------------------------------------------------- closed forms

def check_single_key(attn):
    # N = 1: softmax over one key is 1, so O = V_0 and L = the score itself.
    q, k, v = rnd((2, 3, 5, 64), 1), rnd((2, 3, 1, 64), 2), rnd((2, 3, 1, 64), 3)
    scale = 0.37
    for causal in (False, True):
        o, lse = attn(q, k, v, scale, causal)
        close(o, np.broadcast_to(v.astype(np.float64), o.shape), 1e-15)
        s = scale * np.einsum("bhmd,bhnd->bhmn", q.astype(np.float64), k.astype(np.float64))[..., 0]
        close(lse, s, 1e-12)


def check_constant_scores(attn, N):
    # Q = 0: every score is 0, weights are uniform, O = mean(V) and L = log N.
    # A ragged N catches phantom keys (L would become the log of a padded count).
    q = np.zeros((1, 2, 7, 64), np.float32)
    k, v = rnd((1, 2, N, 64), 4), rnd((1, 2, N, 64), 5)
    o, lse = attn(q, k, v, 0.125, False)
    mean = v.astype(np.float64).mean(axis=2, keepdims=True)
    close(o, np.broadcast_to(mean, o.shape), 1e-14)
    close(lse, math.log(N), 1e-14)


def check_causal_prefix_means(attn):
    # Q = 0, causal, M = N: row i averages V_0..V_i and L_i = log(i+1).
    # A reversed comparison or an excluded diagonal changes both.
    M = N = 150
    q = np.zeros((1, 1, M, 64), np.float32)
    k, v = rnd((1, 1, N, 64), 6), rnd((1, 1, N, 64), 7)
    o, lse = attn(q, k, v, 0.125, True)
    v64 = v.astype(np.float64)[0, 0]
    prefix = np.cumsum(v64, axis=0) / np.arange(1, N + 1)[:, None]
    close(o[0, 0], prefix, 1e-13)
    close(lse[0, 0], np.log(np.arange(1, M + 1)), 1e-14)


def check_causal_row_zero(attn):
    q, k, v = rnd((2, 2, 40, 128), 8), rnd((2, 2, 40, 128), 9), rnd((2, 2, 40, 128), 10)
    scale = 1 / math.sqrt(128)
    o, lse = attn(q, k, v, scale, True)
    close(o[:, :, 0], v[:, :, 0].astype(np.float64), 1e-15)
    s00 = scale * (q[:, :, 0].astype(np.float64) * k[:, :, 0].astype(np.float64)).sum(-1)
    close(lse[:, :, 0], s00, 1e-12)


def check_weights_sum_to_one(attn):
    # V = 1 everywhere: every output element is exactly the sum of the weights.
    q, k = rnd((1, 3, 33, 64), 11, 3.0), rnd((1, 3, 71, 64), 12, 3.0)
    v = np.ones((1, 3, 71, 64), np.float32)
    for causal in (False, True):
        o, _ = attn(q, k, v, 0.125, causal)
        close(o, 1.0, 1e-14)


def check_identity_values(attn):
    # N = D and V = I: O is the probability matrix itself; compare with
    # scipy's softmax of scores built by numpy (M != N exposes a transpose).
    from scipy.special import softmax
    M, N = 48, 64
    q, k = rnd((1, 1, M, 64), 13), rnd((1, 1, N, 64), 14)
    v = np.eye(N, dtype=np.float32)[None, None]
    scale = 0.21
    o, _ = attn(q, k, v, scale, False)
    s = scale * (q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T)
    close(o[0, 0], softmax(s, axis=-1), 1e-15)


def check_large_magnitude_two_keys(attn):
    # q = 8 e0, k0 = 96 e0, k1 = 95 e0, scale 1/8: scores (96, 95), so
    # p = (1, e^-1)/(1 + e^-1) and L = 96 + log(1 + e^-1).
    D = 64
    q = np.zeros((1, 1, 1, D), np.float32); q[..., 0] = 8
    k = np.zeros((1, 1, 2, D), np.float32); k[0, 0, 0, 0] = 96; k[0, 0, 1, 0] = 95
    v = rnd((1, 1, 2, D), 15)
    o, lse = attn(q, k, v, 1 / 8, False)
    p0 = 1 / (1 + math.exp(-1))
    p1 = math.exp(-1) / (1 + math.exp(-1))
    close(o[0, 0, 0], p0 * v[0, 0, 0].astype(np.float64) + p1 * v[0, 0, 1].astype(np.float64), 1e-14)
    assert abs(lse[0, 0, 0] - (96 + math.log1p(math.exp(-1)))) < 1e-13


def check_geometric_scores(attn, c):
    # s_j = c*j (q parallel to k_j = j*u): l = sum_j e^{c(j-(N-1))} is a
    # geometric series, L = c(N-1) + log l, and with V_j = j in column 0,
    # O_0 = sum_j j e^{cj} / sum_j e^{cj}.
    N, D = 200, 64
    q = np.zeros((1, 1, 1, D), np.float32); q[..., 0] = 1.0
    k = np.zeros((1, 1, N, D), np.float32); k[0, 0, :, 0] = np.arange(N)
    v = np.zeros((1, 1, N, D), np.float32); v[0, 0, :, 0] = np.arange(N); v[0, 0, :, 1] = 1.0
    o, lse = attn(q, k, v, c, False)
    r = math.exp(-c)
    l = (1 - r ** N) / (1 - r)
    assert abs(lse[0, 0, 0] - (c * (N - 1) + math.log(l))) < 1e-12
    num = sum((N - 1 - t) * r ** t for t in range(N))
    assert abs(o[0, 0, 0, 0] - num / l) < 1e-11
    assert abs(o[0, 0, 0, 1] - 1.0) < 1e-14


# ------------------------------------------------------------------ invariants

def check_key_shift(attn):
    # K -> K + 1 u^T adds scale*q_i.u to every score of row i: O unchanged,
    # L_i grows by exactly that amount.  Small integers keep the shift exact.
    g = np.random.default_rng(20)
    q = g.integers(-3, 4, (1, 1, 20, 64)).astype(np.float32)
    k = g.integers(-3, 4, (1, 1, 25, 64)).astype(np.float32)
    v = rnd((1, 1, 25, 64), 21)
    u = g.integers(-2, 3, (64,)).astype(np.float32)
    scale = 0.0625
    for causal in (False, True):
        o1, l1 = attn(q, k, v, scale, causal)
        o2, l2 = attn(q, k + u, v, scale, causal)
        close(o1, o2, 1e-12)
        close(l2 - l1, scale * (q[0, 0].astype(np.float64) @ u.astype(np.float64))[None, None], 1e-12)


def check_joint_key_permutation(attn):
    q, k, v = rnd((2, 1, 17, 64), 22), rnd((2, 1, 50, 64), 23), rnd((2, 1, 50, 64), 24)
    perm = np.random.default_rng(25).permutation(50)
    o1, l1 = attn(q, k, v, 0.3, False)
    o2, l2 = attn(q, k[:, :, perm], v[:, :, perm], 0.3, False)
    close(o1, o2, 1e-13)
    close(l1, l2, 1e-13)


def check_linear_in_values(attn):
    q, k = rnd((1, 2, 21, 64), 26), rnd((1, 2, 33, 64), 27)
    g = np.random.default_rng(28)
    # small dyadic values, so a*v + b*w is exact in float32
    v = (g.integers(-64, 65, (1, 2, 33, 64)) / 8).astype(np.float32)
    w = (g.integers(-64, 65, (1, 2, 33, 64)) / 8).astype(np.float32)
    a, b = 0.5, -2.0
    for causal in (False, True):
        ov, lv = attn(q, k, v, 0.125, causal)
        ow, lw = attn(q, k, w, 0.125, causal)
        oc, lc = attn(q, k, (a * v + b * w).astype(np.float32), 0.125, causal)
        close(oc, a * ov + b * ow, 1e-13)
        close(lc, lv, 0)


def check_slices_independent(attn):
    q, k, v = rnd((2, 3, 19, 64), 30), rnd((2, 3, 23, 64), 31), rnd((2, 3, 23, 64), 32)
    o, lse = attn(q, k, v, 0.2, True)
    for b in range(2):
        for h in range(3):
            o1, l1 = attn(q[b:b + 1, h:h + 1].copy(), k[b:b + 1, h:h + 1].copy(), v[b:b + 1, h:h + 1].copy(), 0.2, True)
            np.testing.assert_array_equal(o[b, h], o1[0, 0])
            np.testing.assert_array_equal(lse[b, h], l1[0, 0])


# ------------------------------------------------------ grouped-query heads

def check_gqa_equals_expanded_heads(attn):
    # Query head h reads K/V head h // G: giving every query head its own copy
    # of that K/V head must not change anything.
    for Hk in (1, 2, 3):
        q = rnd((2, 6, 21, 64), 60 + Hk)
        k, v = rnd((2, Hk, 33, 64), 61 + Hk), rnd((2, Hk, 33, 64), 62 + Hk)
        G = 6 // Hk
        for causal in (False, True):
            o, lse = attn(q, k, v, 0.3, causal)
            o2, l2 = attn(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.3, causal)
            np.testing.assert_array_equal(o, o2)
            np.testing.assert_array_equal(lse, l2)


def check_mqa_constant_scores(attn):
    # One K/V head for all query heads and Q = 0: every head of batch b
    # returns the mean of V[b, 0] and L = log N.
    q = np.zeros((2, 4, 5, 64), np.float32)
    k, v = rnd((2, 1, 29, 64), 63), rnd((2, 1, 29, 64), 64)
    o, lse = attn(q, k, v, 0.125, False)
    mean = v.astype(np.float64).mean(axis=2, keepdims=True)  # [2, 1, 1, 64]
    close(o, np.broadcast_to(mean, o.shape), 1e-14)
    close(lse, math.log(29), 1e-14)


def check_gqa_torch(attn):
    # torch fp64 SDPA on K/V expanded with repeat_interleave along heads
    q = rnd((1, 8, 40, 64), 65)
    k, v = rnd((1, 2, 50, 64), 66), rnd((1, 2, 50, 64), 67)
    o, lse = attn(q, k, v, 0.125, True)
    ke = torch.from_numpy(k).repeat_interleave(4, dim=1).numpy()
    ve = torch.from_numpy(v).repeat_interleave(4, dim=1).numpy()
    o_ref, l_ref = torch_reference(q, ke, ve, 0.125, True)
    close(o, o_ref, 1e-12)
    close(lse, l_ref, 1e-12)


# --------------------------------------------------------- library special case

def torch_reference(q, k, v, scale, causal):
    """torch CPU fp64: SDPA for O and logsumexp of the masked scores for L,
    the reference of the pages' Triton test harness, with the top-left causal
    mask spelled out (so it also holds for M != N)."""
    q64, k64, v64 = (torch.from_numpy(np.asarray(x, dtype=np.float64)) for x in (q, k, v))
    M, N = q64.shape[-2], k64.shape[-2]
    mask = torch.ones(M, N, dtype=torch.bool).tril() if causal else None
    o = torch.nn.functional.scaled_dot_product_attention(q64, k64, v64, attn_mask=mask, scale=scale)
    s = (q64 @ k64.transpose(-1, -2)) * scale
    if causal:
        s = s.masked_fill(~mask, float("-inf"))
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


# (batch, n_queries, n_keys, head_dim) shapes of the pages' harnesses at the
# head dims this library supports, plus non-square causal cases.
LIB_SHAPES = [(4, 128, 128, 64), (2, 100, 100, 64), (1, 37, 53, 64), (1, 200, 96, 128),
              (1, 53, 37, 64), (2, 256, 256, 128)]


def check_torch(attn, B, M, N, D, causal):
    q, k, v = rnd((B, 2, M, D), 40 + M), rnd((B, 2, N, D), 41 + N), rnd((B, 2, N, D), 42 + D)
    scale = 1 / math.sqrt(D)
    o, lse = attn(q, k, v, scale, causal)
    o_ref, l_ref = torch_reference(q, k, v, scale, causal)
    close(o, o_ref, 1e-12)
    close(lse, l_ref, 1e-12)


# ------------------------------------------------------------------ brute force

def brute_force(q, k, v, scale, causal, digits=50):
    """Direct evaluation of the definition with 50-digit decimals (no max
    subtraction, no tiling): O = sum_j exp(s_j) v_j / sum_j exp(s_j),
    L = ln sum_j exp(s_j)."""
    ctx = decimal.Context(prec=digits)
    B, H, M, D = q.shape
    N = k.shape[2]
    O = np.zeros((B, H, M, D))
    L = np.zeros((B, H, M))
    sc = decimal.Decimal(float(scale))
    Dec = decimal.Decimal
    for b in range(B):
        for h in range(H):
            for i in range(M):
                J = list(range(min(i + 1, N))) if causal else list(range(N))
                w = []
                for j in J:
                    dot = Dec(0)
                    for d in range(D):
                        dot = ctx.add(dot, ctx.multiply(Dec(float(q[b, h, i, d])), Dec(float(k[b, h, j, d]))))
                    w.append(ctx.exp(ctx.multiply(sc, dot)))
                tot = Dec(0)
                for wj in w:
                    tot = ctx.add(tot, wj)
                L[b, h, i] = float(ctx.ln(tot))
                for d in range(D):
                    acc = Dec(0)
                    for wj, j in zip(w, J):
                        acc = ctx.add(acc, ctx.multiply(wj, Dec(float(v[b, h, j, d]))))
                    O[b, h, i, d] = float(ctx.divide(acc, tot))
    return O, L


BRUTE_CASES = [(5, 8, 8, False), (8, 8, 4, True), (3, 7, 6, True), (8, 3, 5, True)]


def check_brute(attn, M, N, D, causal):
    q, k, v = rnd((1, 2, M, D), 50 + M, 2.0), rnd((1, 2, N, D), 51 + N, 2.0), rnd((1, 2, N, D), 52 + D)
    scale = 0.35
    o, lse = attn(q, k, v, scale, causal)
    ob, lb = brute_force(q, k, v, scale, causal)
    close(o, ob, 1e-13)
    close(lse, lb, 1e-13)


# ------------------------------------------------------------ sliding window

def window_bounds(i, N, causal, wl, wr):
    """First and last key row i sees (lo > hi: none), written out from the
    statement of the window: i - wl <= j <= i + wr, j <= i when causal."""
    lo = 0 if wl < 0 else max(0, i - wl)
    hi = N - 1
    if causal:
        hi = min(hi, i)
    if wr >= 0:
        hi = min(hi, i + wr)
    return lo, hi


WINDOWS = [((2, 1), False), ((0, 0), False), ((3, -1), False), ((-1, 2), False), ((1, 5), True),
           ((4, -1), True), ((2, -1), False)]


def check_window_constant_scores(attn):
    # Q = 0: uniform weights over each row's window, so O is the mean of the
    # window's V rows and L the log of its size; M > N leaves the last rows
    # of the (2, -1) window empty (O = 0, L = -inf).
    M, N = 20, 8
    q = np.zeros((1, 2, M, 64), np.float32)
    k, v = rnd((1, 2, N, 64), 80), rnd((1, 2, N, 64), 81)
    v64 = v.astype(np.float64)
    for (wl, wr), causal in WINDOWS:
        o, lse = attn(q, k, v, 0.125, causal, window=(wl, wr))
        for i in range(M):
            lo, hi = window_bounds(i, N, causal, wl, wr)
            if hi < lo:
                close(o[:, :, i], 0.0, 0)
                assert np.all(lse[:, :, i] == -np.inf)
            else:
                close(o[:, :, i], v64[:, :, lo:hi + 1].mean(axis=2), 1e-14)
                close(lse[:, :, i], math.log(hi - lo + 1), 1e-14)


def check_window_torch(attn):
    # torch fp64 SDPA with the band mask spelled out (rows non-empty)
    M, N = 45, 60
    q, k, v = rnd((1, 2, M, 64), 82), rnd((1, 2, N, 64), 83), rnd((1, 2, N, 64), 84)
    for (wl, wr), causal in [((7, 3), False), ((16, -1), True), ((-1, 5), False), ((0, 0), False)]:
        o, lse = attn(q, k, v, 0.125, causal, window=(wl, wr))
        mask = torch.zeros(M, N, dtype=torch.bool)
        for i in range(M):
            lo, hi = window_bounds(i, N, causal, wl, wr)
            mask[i, lo:hi + 1] = True
        q64, k64, v64 = (torch.from_numpy(x.astype(np.float64)) for x in (q, k, v))
        o_ref = torch.nn.functional.scaled_dot_product_attention(q64, k64, v64, attn_mask=mask, scale=0.125)
        s = (q64 @ k64.transpose(-1, -2) * 0.125).masked_fill(~mask, float("-inf"))
        close(o, o_ref.numpy(), 1e-12)
        close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12)


def check_window_limits(attn):
    # an unbounded window is no window; a right bound of 0 is the causal mask;
    # bounds past the sequence change nothing
    q, k, v = rnd((1, 2, 30, 64), 85), rnd((1, 2, 41, 64), 86), rnd((1, 2, 41, 64), 87)
    o0, l0 = attn(q, k, v, 0.2, False)
    oc, lc = attn(q, k, v, 0.2, True)
    for window, causal, (oe, le) in [((-1, -1), False, (o0, l0)), ((100, 100), False, (o0, l0)),
                                     ((-1, 0), False, (oc, lc)), ((100, 0), False, (oc, lc)),
                                     ((100, 7), True, (oc, lc))]:
        o, lse = attn(q, k, v, 0.2, causal, window=window)
        np.testing.assert_array_equal(o, oe)
        np.testing.assert_array_equal(lse, le)


def brute_force_window(q, k, v, scale, causal, wl, wr, digits=50):
    """The 50-digit brute force over each row's window."""
    B, H, M, D = q.shape
    N = k.shape[2]
    O = np.zeros((B, H, M, D))
    L = np.zeros((B, H, M))
    for i in range(M):
        lo, hi = window_bounds(i, N, causal, wl, wr)
        ob, lb = brute_force(q[:, :, i:i + 1], k[:, :, lo:hi + 1], v[:, :, lo:hi + 1], scale, False, digits)
        O[:, :, i] = ob[:, :, 0]
        L[:, :, i] = lb[:, :, 0]
    return O, L


def check_window_brute(attn):
    q, k, v = rnd((1, 1, 7, 6), 88, 2.0), rnd((1, 1, 9, 6), 89, 2.0), rnd((1, 1, 9, 6), 90)
    for (wl, wr), causal in [((2, 1), False), ((1, -1), True)]:
        o, lse = attn(q, k, v, 0.35, causal, window=(wl, wr))
        ob, lb = brute_force_window(q, k, v, 0.35, causal, wl, wr)
        close(o, ob, 1e-13)
        close(lse, lb, 1e-13)


# ---------------------------------------------------------------- the pytests

def test_window_constant_scores():
    check_window_constant_scores(oracle.attention)


def test_window_matches_torch_band_mask():
    check_window_torch(oracle.attention)


def test_window_limits():
    check_window_limits(oracle.attention)


def test_window_matches_decimal_brute_force():
    check_window_brute(oracle.attention)


def test_varlen_equals_dense_per_sequence():
    # packed head-major sequences of different lengths: each sequence equals
    # the dense oracle on its own rows; a sequence with no keys gives O = 0,
    # L = -inf; an empty sequence is skipped
    lens_q, lens_k = [5, 0, 17, 9], [7, 3, 17, 0]
    cq, ck = np.cumsum([0] + lens_q), np.cumsum([0] + lens_k)
    q, k, v = rnd((3, cq[-1], 64), 91), rnd((1, ck[-1], 64), 92), rnd((1, ck[-1], 64), 93)
    for causal, window in [(False, (-1, -1)), (True, (-1, -1)), (False, (3, 2))]:
        o, lse = oracle.attention_varlen(q, k, v, cq, ck, 0.125, causal, window)
        for b in range(4):
            q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
            if q1 == q0:
                continue
            if k1 == k0:
                assert np.all(o[:, q0:q1] == 0) and np.all(lse[:, q0:q1] == -np.inf)
                continue
            ob, lb = oracle.attention(q[None, :, q0:q1], np.repeat(k[None, :, k0:k1], 3, 1),
                                      np.repeat(v[None, :, k0:k1], 3, 1), 0.125, causal, window=window)
            np.testing.assert_array_equal(o[:, q0:q1], ob[0])
            np.testing.assert_array_equal(lse[:, q0:q1], lb[0])


def test_single_key_gives_value_row_and_score():
    check_single_key(oracle.attention)


@pytest.mark.parametrize("N", [1, 2, 37, 64, 65, 300])
def test_constant_scores_give_mean_and_log_n(N):
    check_constant_scores(oracle.attention, N)


def test_constant_scores_causal_prefix_means():
    check_causal_prefix_means(oracle.attention)


def test_causal_row_zero_sees_only_key_zero():
    check_causal_row_zero(oracle.attention)


def test_weights_sum_to_one():
    check_weights_sum_to_one(oracle.attention)


def test_identity_values_return_softmax_rows():
    check_identity_values(oracle.attention)


def test_large_magnitude_two_keys():
    check_large_magnitude_two_keys(oracle.attention)


@pytest.mark.parametrize("c", [0.05, 0.7])
def test_geometric_scores(c):
    check_geometric_scores(oracle.attention, c)


def test_key_shift_moves_lse_only():
    check_key_shift(oracle.attention)


def test_joint_key_permutation_is_invisible():
    check_joint_key_permutation(oracle.attention)


def test_linear_in_values():
    check_linear_in_values(oracle.attention)


def test_slices_are_independent():
    check_slices_independent(oracle.attention)


@pytest.mark.parametrize("B,M,N,D", LIB_SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_fp64(B, M, N, D, causal):
    check_torch(oracle.attention, B, M, N, D, causal)


def test_matches_torch_on_bf16_inputs():
    # the oracle consumes bf16-rounded inputs exactly (widened to fp32)
    q, k, v = make_inputs(1, 2, 70, 90, 128, "bf16", seed=7, qk_sigma=4.0)
    o, lse = oracle.attention(q, k, v, 1 / math.sqrt(128), False)
    o_ref, l_ref = torch_reference(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                   1 / math.sqrt(128), False)
    close(o, o_ref, 1e-12)
    close(lse, l_ref, 1e-11)


@pytest.mark.parametrize("M,N,D,causal", BRUTE_CASES)
def test_matches_decimal_brute_force(M, N, D, causal):
    check_brute(oracle.attention, M, N, D, causal)


def test_gqa_equals_expanded_heads():
    check_gqa_equals_expanded_heads(oracle.attention)


def test_mqa_constant_scores():
    check_mqa_constant_scores(oracle.attention)


def test_gqa_matches_torch():
    check_gqa_torch(oracle.attention)


def test_fp16_inputs_are_widened_exactly():
    q, k, v = (torch.from_numpy(rnd((1, 2, 30, 64), s)).to(torch.float16) for s in (70, 71, 72))
    o, lse = oracle.attention(q, k, v, 0.125, True)
    o2, l2 = oracle.attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), 0.125, True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)


def test_sampled_rows_equal_full_rows():
    q, k, v = rnd((1, 2, 90, 64), 33), rnd((1, 2, 90, 64), 34), rnd((1, 2, 90, 64), 35)
    rows = np.array([0, 5, 44, 89], np.int64)
    o, lse = oracle.attention(q, k, v, 0.125, True)
    os_, ls_ = oracle.attention(q, k, v, 0.125, True, rows=rows)
    np.testing.assert_array_equal(os_, o[:, :, rows])
    np.testing.assert_array_equal(ls_, lse[:, :, rows])


def test_invalid_arguments_raise():
    q = rnd((1, 1, 4, 64), 36)
    empty = np.zeros((1, 1, 0, 64), np.float32)
    with pytest.raises(ValueError):
        oracle.attention(q, empty, empty, 1.0, False)
    with pytest.raises(ValueError):
        oracle.attention(q, q, q, 1.0, False, rows=np.array([4], np.int64))
    q3 = rnd((1, 3, 4, 64), 37)
    kv2 = rnd((1, 2, 4, 64), 38)
    with pytest.raises(ValueError):  # 3 query heads cannot share 2 K/V heads
        oracle.attention(q3, kv2, kv2, 1.0, False)


# ------------------------------------------------------- planted-mistake check

ALL_PINS = (
    [check_single_key, check_causal_prefix_means, check_causal_row_zero, check_weights_sum_to_one,
     check_identity_values, check_large_magnitude_two_keys, check_key_shift,
     check_joint_key_permutation, check_linear_in_values, check_slices_independent,
     check_gqa_equals_expanded_heads, check_mqa_constant_scores, check_gqa_torch,
     check_window_constant_scores, check_window_torch, check_window_limits, check_window_brute]
    + [lambda a, N=N: check_constant_scores(a, N) for N in (1, 37, 65)]
    + [lambda a, c=c: check_geometric_scores(a, c) for c in (0.05, 0.7)]
    + [lambda a, s=s, c=c: check_torch(a, *s, c) for s in LIB_SHAPES[:4] for c in (False, True)]
    + [lambda a, bc=bc: check_brute(a, *bc) for bc in BRUTE_CASES[:2]]
)

# Text edits of fa2_oracle.c, each a plausible slip.
MUTANTS = {
    "scale dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "log base 2": ("*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    "max missing from L": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "diagonal excluded": ("if (causal && i < hi) hi = i;", "if (causal && i - 1 < hi) hi = i - 1;"),
    "causal reversed": ("if (causal && i < hi) hi = i;", "if (causal && i > lo) lo = i;"),
    "window left bound off by one": ("if (wl >= 0 && i - wl > lo) lo = i - wl;",
                                     "if (wl >= 0 && i - wl + 1 > lo) lo = i - wl + 1;"),
    "window right bound ignored": ("if (wr >= 0 && i + wr < hi) hi = i + wr;", ""),
    "empty window gives L = 0": ("*lse_out = -INFINITY;\n        return;", "*lse_out = 0.0;\n        return;"),
    "no normalisation": ("orow[d] /= l;", "orow[d] /= 1.0;"),
    "weights misaligned with values": ("const double e = s[j];", "const double e = s[n_vis - 1 - j];"),
    "key row misindexed": ("const float* kj = kbh + j * D;", "const float* kj = kbh + (n_vis - 1 - j) * D;"),
    "kv head misindexed": ("const int64_t kvh = b * Hk + h / group;", "const int64_t kvh = b * Hk + h % Hk;"),
    "last key dropped": ("for (int64_t j = 0; j < n_vis; ++j) {\n        s[j] = exp", "for (int64_t j = 0; j + 1 < n_vis; ++j) {\n        s[j] = exp"),
}


def _build_mutant(tmp_path, name, edit):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "fa2_oracle.c")).read()
    old, new = edit
    assert old in src, f"mutant {name!r} no longer applies"
    path = tmp_path / (name.replace(" ", "_") + ".c")
    path.write_text(src.replace(old, new, 1))
    so = str(path) + ".so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(path), "-o", so, "-lm"],
                   check=True)
    import ctypes
    return oracle._bind(ctypes.CDLL(so))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(tmp_path, name):
    lib = _build_mutant(tmp_path, name, MUTANTS[name])

    def mutant(q, k, v, scale, causal, rows=None, window=(-1, -1)):
        return oracle.attention(q, k, v, scale, causal, rows=rows, _lib_override=lib, window=window)

    failures = 0
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except (AssertionError, ValueError, FloatingPointError):
            failures += 1
    assert failures > 0, f"no pin catches the planted mistake {name!r}"


# ------------------------------------------------------------ worked examples

def _golden_ids():
    from tests.golden_cases import load_cases
    return load_cases()


@pytest.mark.parametrize("case", _golden_ids(), ids=lambda c: c["name"])
def test_golden_worked_examples(case):
    from tests.golden_cases import build_case
    q, k, v, scale, causal, o_exp, l_exp = build_case(case)
    o, lse = oracle.attention(q, k, v, scale, causal)
    close(o, o_exp, 1e-12)
    close(lse, l_exp, 1e-12)
