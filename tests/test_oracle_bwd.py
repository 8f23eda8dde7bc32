"""Pins for the oracle's backward pass (runs without a GPU).

The pages print no numbers for the gradients, so the backward oracle is
pinned to what calculus fixes, by routes that share nothing with its chain
rule:

* central finite differences of the oracle's forward (itself pinned in
  ``test_oracle.py``) on inputs whose perturbations are exact in float32;
* torch's fp64 autograd through a materialised softmax, the reference
  backward of "FlashAttention-2 from PyTorch to Triton";
* closed forms: one key (P = 1 gives dQ = dK = 0, dV = sum of dO); zero
  queries (uniform weights, causal prefix weights 1/(i+1));
* invariants: every softmax row's dS sums to zero, so the dK rows of a head
  sum to zero; weights sum to one, so the dV rows sum to the dO rows; the
  scores are bilinear in Q and K, so <Q, dQ> = <K, dK>; O is linear in V, so
  <V, dV> = <O, dO>.

The same pins run against deliberately broken builds of the oracle's backward
(``test_bwd_pins_catch_planted_mistakes``).
"""
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle


def rnd(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal(shape) * scale).astype(np.float32)


def grid_rnd(shape, seed, scale=1.0):
    """Gaussian values rounded to multiples of 2^-8 (at most 12 significant
    bits), so x +- 2^-12 is exact in float32."""
    x = np.round(rnd(shape, seed, scale) * 256.0) / 256.0
    return np.clip(x, -7.0, 7.0).astype(np.float32)


def close(a, b, atol, rtol=0.0):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


# ------------------------------------------------------------ finite differences

def check_finite_differences(bwd, causal, H=2, Hk=1, M=9, N=11, D=8, seed=0, window=(-1, -1)):
    """d/dx sum(O * dO) by central differences of the fp64 forward, at a few
    entries of each of q, k and v."""
    q, k, v = grid_rnd((1, H, M, D), seed), grid_rnd((1, Hk, N, D), seed + 1), grid_rnd((1, Hk, N, D), seed + 2)
    do = rnd((1, H, M, D), seed + 3)
    scale = 0.3
    dq, dk, dv = bwd(q, k, v, do, scale, causal, window=window)
    h = 2.0 ** -12

    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, scale, causal, window=window)
        return float(np.sum(o * do.astype(np.float64)))

    g = np.random.default_rng(seed + 4)
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(g.integers(0, s)) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            assert abs(fd - grad[idx]) <= 2e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


# --------------------------------------------------------------- library case

def band_mask(M, N, causal, wl, wr):
    """Boolean [M, N] mask of the visible pairs, written out from the
    statement of the window (key j visible to row i iff i - wl <= j <= i + wr,
    a side unbounded when -1, and j <= i when causal)."""
    i = torch.arange(M)[:, None]
    j = torch.arange(N)[None, :]
    mask = torch.ones(M, N, dtype=torch.bool)
    if causal:
        mask &= j <= i
    if wl >= 0:
        mask &= j >= i - wl
    if wr >= 0:
        mask &= j <= i + wr
    return mask


def torch_grads(q, k, v, do, scale, causal, window=(-1, -1)):
    """fp64 autograd through a materialised, masked softmax; GQA by repeating
    K/V heads (autograd sums the repeated heads' gradients)."""
    H, Hk = q.shape[1], k.shape[1]
    tq, tk, tv = (torch.from_numpy(x.astype(np.float64)).requires_grad_(True) for x in (q, k, v))
    kk = tk.repeat_interleave(H // Hk, dim=1)
    vv = tv.repeat_interleave(H // Hk, dim=1)
    s = scale * torch.matmul(tq, kk.transpose(-1, -2))
    if causal or window != (-1, -1):
        M, N = q.shape[2], k.shape[2]
        mask = band_mask(M, N, causal, *window)
        s = s.masked_fill(~mask, float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vv)
    o.backward(torch.from_numpy(do.astype(np.float64)))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


LIB_CASES = [  # (B, H, Hk, M, N, D)
    (1, 2, 2, 33, 33, 16),
    (2, 3, 3, 17, 40, 32),
    (1, 4, 2, 50, 30, 16),
    (1, 4, 1, 20, 20, 8),
]


def check_torch(bwd, B, H, Hk, M, N, D, causal, seed=10, window=(-1, -1)):
    q, k, v = rnd((B, H, M, D), seed), rnd((B, Hk, N, D), seed + 1), rnd((B, Hk, N, D), seed + 2)
    do = rnd((B, H, M, D), seed + 3)
    scale = 1 / math.sqrt(D)
    got = bwd(q, k, v, do, scale, causal, window=window)
    ref = torch_grads(q, k, v, do, scale, causal, window)
    for g, r in zip(got, ref):
        close(g, r, 1e-12, 1e-10)


# ---------------------------------------------------------------- closed forms

def check_single_key(bwd):
    # N = 1: every weight is 1, so O = V_0 whatever Q and K are: dQ = dK = 0
    # and dV_0 = the sum of dO over the rows and the heads that read it.
    q, k, v = rnd((2, 4, 6, 16), 20), rnd((2, 2, 1, 16), 21), rnd((2, 2, 1, 16), 22)
    do = rnd((2, 4, 6, 16), 23)
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, 0.4, causal)
        close(dq, 0.0, 1e-15)
        close(dk, 0.0, 1e-15)
        expect = do.astype(np.float64).reshape(2, 2, 2, 6, 16).sum(axis=(2, 3))[:, :, None, :]
        close(dv, expect, 1e-13)


def check_zero_queries(bwd):
    # Q = 0, non-causal: P = 1/N, so dV_j = sum_i dO_i / N;
    # dK = scale * dS^T Q = 0; dQ_i = (scale / N) sum_j <dO_i, V_j - Vbar> K_j.
    M, N, D = 7, 13, 16
    q = np.zeros((1, 1, M, D), np.float32)
    k, v, do = rnd((1, 1, N, D), 24), rnd((1, 1, N, D), 25), rnd((1, 1, M, D), 26)
    scale = 0.25
    dq, dk, dv = bwd(q, k, v, do, scale, False)
    k64, v64, do64 = (x.astype(np.float64)[0, 0] for x in (k, v, do))
    close(dk, 0.0, 1e-15)
    close(dv[0, 0], np.broadcast_to(do64.sum(axis=0) / N, (N, D)), 1e-13)
    vc = v64 - v64.mean(axis=0)
    expect_dq = np.zeros((M, D))
    for i in range(M):
        for j in range(N):
            expect_dq[i] += (scale / N) * float(do64[i] @ vc[j]) * k64[j]
    close(dq[0, 0], expect_dq, 1e-13)


def check_zero_queries_causal(bwd):
    # Q = 0, causal, M = N: row i weights keys 0..i by 1/(i+1), so
    # dV_j = sum_{i >= j} dO_i / (i+1), and row 0 (one key) has dQ_0 = 0.
    M = N = 40
    D = 8
    q = np.zeros((1, 1, M, D), np.float32)
    k, v, do = rnd((1, 1, N, D), 27), rnd((1, 1, N, D), 28), rnd((1, 1, M, D), 29)
    dq, dk, dv = bwd(q, k, v, do, 0.5, True)
    do64 = do.astype(np.float64)[0, 0]
    w = do64 / np.arange(1, M + 1)[:, None]
    expect_dv = np.cumsum(w[::-1], axis=0)[::-1]
    close(dv[0, 0], expect_dv, 1e-13)
    close(dq[0, 0, 0], 0.0, 1e-15)
    close(dk, 0.0, 1e-15)


# ----------------------------------------------------------------- invariants

def check_invariants(bwd, causal, seed=30):
    B, H, Hk, M, N, D = 2, 4, 2, 25, 31, 16
    q, k, v = rnd((B, H, M, D), seed), rnd((B, Hk, N, D), seed + 1), rnd((B, Hk, N, D), seed + 2)
    do = rnd((B, H, M, D), seed + 3)
    scale = 0.3
    dq, dk, dv = bwd(q, k, v, do, scale, causal)
    o, _ = oracle.attention(q, k, v, scale, causal)
    G = H // Hk
    do64 = do.astype(np.float64)
    # dK rows of each K/V head sum to zero (row sums of dS vanish).
    close(dk.sum(axis=2), 0.0, 1e-12)
    # dV rows sum to the dO rows of the heads that read them.
    close(dv.sum(axis=2), do64.reshape(B, Hk, G, M, D).sum(axis=(2, 3)), 1e-12)
    # <Q, dQ> = <K, dK> per K/V head group (both equal sum_ij dS_ij s_ij).
    qdq = (q.astype(np.float64) * dq).reshape(B, Hk, G * M * D).sum(axis=-1)
    kdk = (k.astype(np.float64) * dk).reshape(B, Hk, N * D).sum(axis=-1)
    close(qdq, kdk, 1e-12)
    # <V, dV> = <O, dO> (O is linear in V).
    vdv = (v.astype(np.float64) * dv).reshape(B, Hk, N * D).sum(axis=-1)
    odo = (o * do64).reshape(B, Hk, G * M * D).sum(axis=-1)
    close(vdv, odo, 1e-12)


def check_window_empty_rows(bwd):
    # M > N with a left window of 2: rows 13.. see no key.  They have no
    # gradient (dQ = 0) and their dO adds nothing to dK, dV: the gradients
    # equal those of the problem without those rows.
    M, N, D = 20, 11, 8
    q, k, v, do = rnd((1, 2, M, D), 50), rnd((1, 2, N, D), 51), rnd((1, 2, N, D), 52), rnd((1, 2, M, D), 53)
    dq, dk, dv = bwd(q, k, v, do, 0.3, False, window=(2, -1))
    close(dq[:, :, 13:], 0.0, 0)
    dq2, dk2, dv2 = bwd(q[:, :, :13].copy(), k, v, do[:, :, :13].copy(), 0.3, False, window=(2, -1))
    close(dq[:, :, :13], dq2, 1e-15)
    close(dk, dk2, 1e-15)
    close(dv, dv2, 1e-15)


WINDOW_CASES = [((3, 2), False), ((4, -1), True), ((-1, 3), False), ((0, 0), False)]


def bwd_oracle(q, k, v, do, scale, causal, window=(-1, -1)):
    return oracle.attention_bwd(q, k, v, do, scale, causal, window=window)


ALL_PINS = (
    [check_single_key, check_zero_queries, check_zero_queries_causal]
    + [lambda b, c=c: check_invariants(b, c) for c in (False, True)]
    + [lambda b, c=c: check_finite_differences(b, c) for c in (False, True)]
    + [lambda b, c=c: check_finite_differences(b, c, H=4, Hk=2, M=12, N=7, seed=5) for c in (False, True)]
    + [lambda b, s=s, c=c: check_torch(b, *s, c) for s in LIB_CASES for c in (False, True)]
    + [check_window_empty_rows]
    + [lambda b, w=w, c=c: check_finite_differences(b, c, M=12, N=14, seed=7, window=w) for w, c in WINDOW_CASES]
    + [lambda b, w=w, c=c: check_torch(b, 1, 4, 2, 26, 30, 16, c, window=w) for w, c in WINDOW_CASES]
)


def test_single_key():
    check_single_key(bwd_oracle)


def test_zero_queries():
    check_zero_queries(bwd_oracle)


def test_zero_queries_causal():
    check_zero_queries_causal(bwd_oracle)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    check_invariants(bwd_oracle, causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(2, 1, 9, 11, 0), (4, 2, 12, 7, 5), (3, 3, 16, 16, 9)])
def test_finite_differences(causal, heads):
    H, Hk, M, N, seed = heads
    check_finite_differences(bwd_oracle, causal, H=H, Hk=Hk, M=M, N=N, seed=seed)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", LIB_CASES, ids=lambda s: "x".join(map(str, s)))
def test_matches_torch_autograd(shape, causal):
    check_torch(bwd_oracle, *shape, causal)


def test_window_empty_rows_have_no_gradient():
    check_window_empty_rows(bwd_oracle)


@pytest.mark.parametrize("window,causal", WINDOW_CASES)
def test_window_finite_differences(window, causal):
    check_finite_differences(bwd_oracle, causal, H=4, Hk=2, M=12, N=14, seed=7, window=window)


@pytest.mark.parametrize("window,causal", WINDOW_CASES)
def test_window_matches_torch_autograd(window, causal):
    check_torch(bwd_oracle, 1, 4, 2, 26, 30, 16, causal, window=window)


def test_varlen_backward_equals_per_sequence():
    # packed sequences: each sequence's gradients are the dense oracle's on
    # its own rows; keys of a sequence without queries get zero gradient
    lens_q, lens_k = [6, 0, 13, 9], [8, 5, 13, 0]
    cq, ck = np.cumsum([0] + lens_q), np.cumsum([0] + lens_k)
    q, do = rnd((4, cq[-1], 16), 60), rnd((4, cq[-1], 16), 61)
    k, v = rnd((2, ck[-1], 16), 62), rnd((2, ck[-1], 16), 63)
    for causal, window in [(False, (-1, -1)), (True, (-1, -1)), (False, (3, 1))]:
        dq, dk, dv = oracle.attention_bwd_varlen(q, k, v, do, cq, ck, 0.25, causal, window)
        for b in range(4):
            q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
            if q1 == q0 or k1 == k0:
                close(dq[:, q0:q1], 0.0, 0)
                close(dk[:, k0:k1], 0.0, 0)
                close(dv[:, k0:k1], 0.0, 0)
                continue
            g = oracle.attention_bwd(q[None, :, q0:q1], k[None, :, k0:k1], v[None, :, k0:k1], do[None, :, q0:q1],
                                     0.25, causal, window=window)
            np.testing.assert_array_equal(dq[:, q0:q1], g[0][0])
            np.testing.assert_array_equal(dk[:, k0:k1], g[1][0])
            np.testing.assert_array_equal(dv[:, k0:k1], g[2][0])


def test_bf16_inputs_are_widened_exactly():
    q, k, v, do = (torch.from_numpy(rnd((1, 2, 20, 16), s)).to(torch.bfloat16) for s in (40, 41, 42, 43))
    a = oracle.attention_bwd(q, k, v, do, 0.25, True)
    b = oracle.attention_bwd(*(x.float().numpy() for x in (q, k, v, do)), 0.25, True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_invalid_arguments_raise():
    q = rnd((1, 3, 4, 16), 44)
    kv = rnd((1, 2, 4, 16), 45)
    with pytest.raises(ValueError):  # 3 query heads cannot share 2 K/V heads
        oracle.attention_bwd(q, kv, kv, q, 1.0, False)
    with pytest.raises(ValueError):  # dO must be shaped like Q
        oracle.attention_bwd(q, q, q, q[:, :, :3], 1.0, False)
    empty = np.zeros((1, 3, 0, 16), np.float32)
    with pytest.raises(ValueError):  # no keys
        oracle.attention_bwd(q, empty, empty, q, 1.0, False)


# ------------------------------------------------------- planted-mistake check

MUTANTS = {
    "D term dropped": ("const double ds = p[j] * (dp[j] - Di);", "const double ds = p[j] * dp[j];"),
    "D sign flipped": ("const double ds = p[j] * (dp[j] - Di);", "const double ds = p[j] * (dp[j] + Di);"),
    "dK scale dropped": ("dkj[d] += scale * ds * (double)qi[d];", "dkj[d] += ds * (double)qi[d];"),
    "dQ scale dropped": ("dqi[d] += scale * ds * (double)kj[d];", "dqi[d] += ds * (double)kj[d];"),
    "dQ reads V": ("dqi[d] += scale * ds * (double)kj[d];",
                   "dqi[d] += scale * ds * (double)vbh[j * D + d];"),
    "dK reads dO": ("dkj[d] += scale * ds * (double)qi[d];", "dkj[d] += scale * ds * (double)doi[d];"),
    "dV weighted by dP": ("dvj[d] += p[j] * (double)doi[d];", "dvj[d] += dp[j] * (double)doi[d];"),
    "dV weighted by dS": ("dvj[d] += p[j] * (double)doi[d];", "dvj[d] += ds * (double)doi[d];"),
    "bwd weights unnormalised": ("for (int64_t j = 0; j < n_vis; ++j) p[j] /= l;",
                                 "for (int64_t j = 0; j < n_vis; ++j) p[j] /= 1.0;"),
    "causal reversed": ("if (causal && i < hi) hi = i;", "if (causal && i > lo) lo = i;"),
    "diagonal excluded": ("if (causal && i < hi) hi = i;", "if (causal && i - 1 < hi) hi = i - 1;"),
    "bwd window ignored": ("visible_keys(i, N, causal, wl, wr, &j0, &n_vis); /* (1) */",
                           "visible_keys(i, N, causal, -1, -1, &j0, &n_vis); /* (1) */"),
    "bwd empty row keeps a gradient": ("if (n_vis <= 0) return; /* a row that sees no key has no gradient */",
                                       "if (n_vis <= 0) { n_vis = 1; j0 = 0; }"),
    "bwd visible keys misplaced": ("    kbh += j0 * D;\n    vbh += j0 * D;\n    dkbh += j0 * D;",
                                   "    kbh += j0 * D;\n    vbh += j0 * D;\n    dkbh += 0 * D;"),
    "bwd kv head misindexed": ("const int64_t bh = b * H + hk * group + g;",
                               "const int64_t bh = b * H + g * Hk + hk;"),
    "dP reads K": ("const float* vrow = vbh + j * D;", "const float* vrow = kbh + j * D;"),
}


def _build_mutant(tmp_path, name, edit):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "fa2_oracle.c")).read()
    old, new = edit
    assert src.count(old) == 1, f"mutant {name!r} does not apply to exactly one place"
    path = tmp_path / (name.replace(" ", "_") + ".c")
    path.write_text(src.replace(old, new, 1))
    so = str(path) + ".so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(path), "-o", so, "-lm"],
                   check=True)
    import ctypes
    return oracle._bind(ctypes.CDLL(so))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_pins_catch_planted_mistakes(tmp_path, name):
    lib = _build_mutant(tmp_path, name, MUTANTS[name])

    def mutant(q, k, v, do, scale, causal, window=(-1, -1)):
        return oracle.attention_bwd(q, k, v, do, scale, causal, _lib_override=lib, window=window)

    failures = 0
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except (AssertionError, ValueError, FloatingPointError):
            failures += 1
    assert failures > 0, f"no pin catches the planted mistake {name!r}"
