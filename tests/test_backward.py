"""Parity of the backward pass (fa2_bwd, through the C ABI) with the fp64
CPU oracle.

Tolerance.  The kernels round four things the oracle keeps exact: the
forward output O (stored in the I/O dtype, it enters delta = rowsum(dO o O)),
P and dS (rounded once to 16 bits as MFMA operands), and dQ, dK, dV
themselves.  Replaying exactly those roundings in fp64 on N(0,1) and
N(0,4^2) inputs (D = 64 and 128, causal and not, M, N up to 1024) gives a
max-abs error of at most 7.9e-3 (bf16) and 8.1e-4 (fp16) times the largest
|gradient| of the tensor.  The bound checked here is 2e-2 (bf16) and 2.5e-3
(fp16) times max(max|reference|, 0.1) per tensor: about 2.5x the replayed
error, and the 0.1 floor keeps tensors whose exact gradient vanishes (one key:
dS = 0) at a small absolute bound instead of zero.

fp32 keeps every product in fp32 (P and dS included), so what remains is
fp32 rounding in the length-D dot products and the sums over rows, and the
cancellation in dP - Delta (two O(sqrt(D)) dot products that agree to a few
ulp when a row's weight sits on few keys).  Observed errors on these cases
stay below 7e-5 times max(max|reference|, 1); the bound is 1e-4 times
max(max|reference|, 1): the floor 1 is the size of a gradient of N(0,1)
inputs, and the cancellation leaves an absolute error of order 1e-5 even
where the exact gradient vanishes (one key).
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_23_amd as fa2
import oracle
import workloads
from tests.test_parity import note

pytestmark = pytest.mark.gpu

TOL_BWD = {"bf16": 2e-2, "f16": 2.5e-3, "f32": 1e-4}
FLOOR = {"bf16": 0.1, "f16": 0.1, "f32": 1.0}


def run_bwd(q, k, v, do, causal, scale=None):
    """Forward then backward on the GPU; returns float64 numpy dq, dk, dv."""
    dev = [t.to("cuda") for t in (q, k, v, do)]
    o, lse = fa2.forward(dev[0], dev[1], dev[2], causal=causal, scale=scale)
    dq, dk, dv = fa2.backward(dev[0], dev[1], dev[2], o, lse, dev[3], causal=causal, scale=scale)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))


def compare_grads(got, ref, dtype, what):
    tol = TOL_BWD[dtype]
    errs = []
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert g.shape == r.shape, f"{what}: {name} shape {g.shape} != {r.shape}"
        assert np.isfinite(g).all(), f"{what}: non-finite {name}"
        if g.size == 0:
            errs.append(0.0)
            continue
        err = float(np.abs(g - r).max())
        bound = tol * max(float(np.abs(r).max()), FLOOR[dtype])
        errs.append(err)
        assert err <= bound, f"{what}: {name} error {err:.3e} > {bound:.3e}"
    note(f"{what}: max|d(dq)|={errs[0]:.2e} max|d(dk)|={errs[1]:.2e} max|d(dv)|={errs[2]:.2e}")
    return errs


def check(B, H, M, N, D, dtype, causal, Hk=None, seed=0, qk_sigma=1.0):
    what = f"bwd B={B} H={H} Hk={Hk or H} M={M} N={N} D={D} {dtype} causal={causal} sigma={qk_sigma}"
    note("case " + what)
    q, k, v = workloads.make_inputs(B, H, M, N, D, dtype, seed, qk_sigma, Hk=Hk)
    do = workloads.make_dout(B, H, M, D, dtype, seed)
    got = run_bwd(q, k, v, do, causal)
    ref = oracle.attention_bwd(q, k, v, do, 1.0 / math.sqrt(D), causal)
    return compare_grads(got, ref, dtype, what)


# shapes span several query tiles (64 rows), key tiles (128 keys per dK/dV
# workgroup, 32 / 64 per dQ tile) and ragged tails on both sides
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("M,N", [(300, 300), (200, 517), (513, 64), (64, 1000), (257, 129)])
def test_backward_parity(M, N, D, causal, dtype):
    check(2, 2, M, N, D, dtype, causal, seed=M + 3 * N + D)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H,Hk", [(8, 2), (6, 1), (4, 4)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_grouped_query_heads(dtype, H, Hk, D, causal):
    # dK, dV of a K/V head sum over its query heads
    check(2, H, 333, 290, D, dtype, causal, Hk=Hk, seed=H * 10 + Hk)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_large_scores(causal, dtype):
    # Q, K ~ N(0, 4^2): near one-hot softmax rows, scores far past exp's range
    check(2, 2, 250, 700, 64, dtype, causal, seed=11, qk_sigma=4.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("M,N", [(1, 1), (1, 700), (700, 1), (2, 3), (33, 31)])
def test_backward_small_and_degenerate(M, N, causal, dtype):
    check(1, 3, M, N, 128, dtype, causal, seed=M * 1000 + N)


def test_backward_no_query_rows_gives_zero_kv_grads():
    q = torch.zeros((2, 4, 0, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.randn((2, 2, 77, 64), device="cuda").to(torch.bfloat16)
    v = torch.randn((2, 2, 77, 64), device="cuda").to(torch.bfloat16)
    o = torch.zeros_like(q)
    lse = torch.zeros((2, 4, 0), dtype=torch.float32, device="cuda")
    dk = torch.full_like(k, 3.0)
    dv = torch.full_like(v, 3.0)
    dq, dk, dv = fa2.backward(q, k, v, o, lse, torch.zeros_like(q), dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert dq.numel() == 0
    assert (dk == 0).all() and (dv == 0).all()


def test_causal_keys_past_the_last_query_get_zero_grads():
    # top-left causal with N > M: keys j >= M are visible to no query
    M, N = 100, 300
    q, k, v = workloads.make_inputs(1, 2, M, N, 64, "bf16", 21)
    do = workloads.make_dout(1, 2, M, 64, "bf16", 21)
    _, dk, dv = run_bwd(q, k, v, do, True)
    assert (dk[:, :, M:] == 0).all() and (dv[:, :, M:] == 0).all()
    assert np.abs(dk[:, :, :M]).max() > 0


def test_backward_is_deterministic():
    q, k, v = workloads.make_inputs(2, 8, 700, 700, 128, "bf16", 31, Hk=2)
    do = workloads.make_dout(2, 8, 700, 128, "bf16", 31)
    a = run_bwd(q, k, v, do, True)
    b = run_bwd(q, k, v, do, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_autograd_function_matches_backward():
    q, k, v = workloads.make_inputs(1, 4, 200, 333, 64, "bf16", 41, Hk=2)
    do = workloads.make_dout(1, 4, 200, 64, "bf16", 41)
    qd, kd, vd = (t.to("cuda").requires_grad_(True) for t in (q, k, v))
    out = fa2.attention(qd, kd, vd, causal=False)
    out.backward(do.to("cuda"))
    torch.cuda.synchronize()
    ref = run_bwd(q, k, v, do, False)
    for t, r in zip((qd.grad, kd.grad, vd.grad), ref):
        assert np.array_equal(t.float().cpu().numpy().astype(np.float64), r)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backward_rejects_unsupported_head_dim(dtype):
    lse = torch.zeros((1, 1, 8), device="cuda")
    q = torch.zeros((1, 1, 8, 96), dtype=dtype, device="cuda")
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.backward(q, q.clone(), q.clone(), q.clone(), lse, q.clone())
    assert e.value.status == fa2.FA2_ERR_UNSUPPORTED


def test_backward_full_size_causal_4k_sampled_heads():
    # the causal bf16 4k workload at its full size on the GPU; two (b, h)
    # slices recomputed by the oracle (its backward runs one thread per slice)
    w = workloads.get("causal_bf16_4k")
    note(f"case bwd full size {w.describe()}")
    q, k, v = workloads.workload_inputs(w)
    do = workloads.make_dout(w.B, w.H, w.M, w.D, w.dtype, w.seed)
    got = run_bwd(q, k, v, do, w.causal)
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        sl = slice(b, b + 1), slice(h, h + 1)
        ref = oracle.attention_bwd(q[sl], k[sl], v[sl], do[sl], w.scale, w.causal)
        compare_grads([g[sl] for g in got], ref, w.dtype, f"full-size causal 4k slice b={b} h={h}")


# --------------------------------------------- sliding window and packed sequences

BWD_WINDOWS = [((16, 16), False), ((100, 0), False), ((70, -1), True), ((-1, 40), False), ((0, 0), False)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("M,N", [(300, 300), (200, 517), (700, 130)])
@pytest.mark.parametrize("window,causal", BWD_WINDOWS)
def test_backward_sliding_window(window, causal, M, N, D, dtype):
    what = f"bwd local B=2 H=4 Hk=2 M={M} N={N} D={D} {dtype} causal={causal} window={window}"
    note("case " + what)
    q, k, v = workloads.make_inputs(2, 4, M, N, D, dtype, seed=M + N + D, Hk=2)
    do = workloads.make_dout(2, 4, M, D, dtype, seed=M + N)
    dev = [t.to("cuda") for t in (q, k, v, do)]
    o, lse = fa2.forward(dev[0], dev[1], dev[2], causal=causal, window=window)
    grads = fa2.backward(dev[0], dev[1], dev[2], o, lse, dev[3], causal=causal, window=window)
    torch.cuda.synchronize()
    got = tuple(t.float().cpu().numpy().astype(np.float64) for t in grads)
    ref = oracle.attention_bwd(q, k, v, do, 1.0 / math.sqrt(D), causal, window=window)
    compare_grads(got, ref, dtype, what)


def test_autograd_function_with_window():
    q, k, v = workloads.make_inputs(1, 2, 180, 180, 128, "bf16", 51)
    do = workloads.make_dout(1, 2, 180, 128, "bf16", 51)
    qd, kd, vd = (t.to("cuda").requires_grad_(True) for t in (q, k, v))
    out = fa2.attention(qd, kd, vd, causal=True, window=(50, -1))
    out.backward(do.to("cuda"))
    torch.cuda.synchronize()
    got = tuple(t.grad.float().cpu().numpy().astype(np.float64) for t in (qd, kd, vd))
    ref = oracle.attention_bwd(q, k, v, do, 1.0 / math.sqrt(128), True, window=(50, -1))
    compare_grads(got, ref, "bf16", "autograd with window (50, -1) causal")


PACKED = [
    ([1, 129, 0, 300, 64, 257], [1, 129, 0, 300, 64, 257]),
    ([17, 250, 64, 1], [300, 3, 129, 700]),
    ([40, 90, 7], [0, 120, 33]),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lens", PACKED, ids=["self", "cross", "nokeys"])
@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (20, 3))])
def test_backward_varlen(causal, window, lens, D, dtype):
    lens_q, lens_k = lens
    what = f"bwd varlen H=4 Hk=2 D={D} {dtype} causal={causal} window={window} lens_q={lens_q} lens_k={lens_k}"
    note("case " + what)
    cq = np.cumsum([0] + lens_q).astype(np.int32)
    ck = np.cumsum([0] + lens_k).astype(np.int32)
    q, _, _ = workloads.make_inputs(1, 4, int(cq[-1]), 1, D, dtype, seed=sum(lens_q) + D)
    _, k, v = workloads.make_inputs(1, 2, 1, int(ck[-1]), D, dtype, seed=sum(lens_k) + D + 1)
    do = workloads.make_dout(1, 4, int(cq[-1]), D, dtype, seed=sum(lens_q))
    q, k, v, do = q[0].contiguous(), k[0].contiguous(), v[0].contiguous(), do[0].contiguous()
    dev = [t.to("cuda") for t in (q, k, v, do)]
    cqd, ckd = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    o, lse = fa2.forward_varlen(dev[0], dev[1], dev[2], cqd, ckd, max(lens_q), causal=causal, window=window)
    grads = fa2.backward_varlen(dev[0], dev[1], dev[2], o, lse, dev[3], cqd, ckd, max(lens_q), max(lens_k),
                                causal=causal, window=window)
    torch.cuda.synchronize()
    got = tuple(t.float().cpu().numpy().astype(np.float64) for t in grads)
    ref = oracle.attention_bwd_varlen(q, k, v, do, cq, ck, 1.0 / math.sqrt(D), causal, window)
    compare_grads(got, ref, dtype, what)


# Delta, the row correction of dS = P (dP - Delta), is part of fa2_bwd's
# output: rowsum(dO o O) over the O the forward stored.  For 16-bit inputs the
# dQ kernel computes it (from the dO it holds and one read of O) and stores it
# for the dK/dV kernel; fp32 has a kernel of its own.  Every row must be
# written (the buffer starts as NaN), and each value is a fp32 sum of D exact
# products, so it is within D ulps of the fp64 sum of their magnitudes.
@pytest.mark.parametrize("dtype,D,causal,H,Hk,M,N,window", [
    ("bf16", 128, True, 4, 4, 300, 300, (-1, -1)),
    ("bf16", 64, False, 6, 2, 257, 129, (-1, -1)),
    ("f16", 128, False, 2, 1, 77, 500, (-1, -1)),
    ("bf16", 128, True, 2, 2, 333, 333, (40, 0)),
    ("f32", 64, True, 2, 2, 130, 130, (-1, -1)),
])
def test_backward_writes_delta_as_rowsum_dout_o(dtype, D, causal, H, Hk, M, N, window):
    what = f"delta {dtype} D={D} causal={causal} H={H} Hk={Hk} M={M} N={N} window={window}"
    note("case " + what)
    B = 2
    q, k, v = workloads.make_inputs(B, H, M, N, D, dtype, 11, 1.0, Hk=Hk)
    do = workloads.make_dout(B, H, M, D, dtype, 11)
    q, k, v, do = (t.to("cuda") for t in (q, k, v, do))
    o, lse = fa2.forward(q, k, v, causal=causal, window=window)
    delta = torch.full((B, H, M), float("nan"), dtype=torch.float32, device="cuda")
    fa2.backward(q, k, v, o, lse, do, causal=causal, delta=delta, window=window)
    torch.cuda.synchronize()
    o64 = o.float().cpu().numpy().astype(np.float64)
    do64 = do.float().cpu().numpy().astype(np.float64)
    ref = (o64 * do64).sum(axis=-1)
    mag = np.abs(o64 * do64).sum(axis=-1)
    got = delta.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all(), f"{what}: rows of delta not written"
    err = np.abs(got - ref)
    bound = D * 2.0 ** -23 * mag + 1e-30
    assert (err <= bound).all(), f"{what}: max excess {float((err - bound).max()):.3e}"
    note(f"{what}: max|d delta|={float(err.max()):.2e}")
