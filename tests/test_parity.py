"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Tolerances (max-abs over every checked element, O and L separately):
  fp32 I/O: 1e-4 on O and on L;
  bf16 I/O: 2e-2 on O and 1e-3 on L;
  fp16 I/O: 5e-3 on O and 1e-3 on L (8x finer rounding than bf16 for P and
            O; L goes through the same fp32 path as bf16),
where the oracle consumes exactly the rounded inputs the kernel sees.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.golden_cases import build_case, load_cases

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-3), "f16": (5e-3, 1e-3)}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(q, k, v, causal, scale=None):
    import exact_attention_23_amd as fa2
    dq, dk, dv = (t.to("cuda") for t in (q, k, v))
    o, lse = fa2.forward(dq, dk, dv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(o, lse, o_ref, l_ref, dtype, what):
    tol_o, tol_l = TOL[dtype]
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    err_o = float(np.abs(o - o_ref).max()) if o.size else 0.0
    err_l = float(np.abs(lse - l_ref).max()) if lse.size else 0.0
    note(f"{what}: max|dO|={err_o:.3e} (tol {tol_o}), max|dL|={err_l:.3e} (tol {tol_l})")
    assert err_o <= tol_o, f"{what}: O error {err_o} > {tol_o}"
    assert err_l <= tol_l, f"{what}: L error {err_l} > {tol_l}"
    return err_o, err_l


def check_case(B, H, M, N, D, dtype, causal, seed=0, qk_sigma=1.0, v_sigma=1.0, rows=None):
    what = f"B={B} H={H} M={M} N={N} D={D} {dtype} causal={causal} seed={seed}"
    note("case " + what)
    q, k, v = workloads.make_inputs(B, H, M, N, D, dtype, seed, qk_sigma, v_sigma)
    scale = 1.0 / math.sqrt(D)
    o, lse = run_gpu(q, k, v, causal)
    o_ref, l_ref = oracle.attention(q, k, v, scale, causal, rows=rows)
    if rows is not None:
        o, lse = o[:, :, rows], lse[:, :, rows]
    return compare(o, lse, o_ref, l_ref, dtype, what)


# ------------------------------------------------------------- the workloads

@pytest.mark.parametrize("name", workloads.ORDER)
def test_workload_parity(name):
    w = workloads.get(name)
    rows = workloads.sample_rows(w)
    rows = None if rows is None else rows.numpy()
    check_case(w.B, w.H, w.M, w.N, w.D, w.dtype, w.causal, w.seed, w.qk_sigma, w.v_sigma, rows=rows)


@pytest.mark.parametrize("name", workloads.WIDENED)
def test_widened_workload_parity(name):
    # grouped-query heads, fp16, split K/V, sliding window and packed
    # sequences at the measured sizes, through the entry point the bench uses
    import exact_attention_23_amd as fa2
    w = workloads.get(name)
    note("case " + w.describe() + f" n_splits={w.n_splits} window={w.window}")
    q, k, v = workloads.workload_inputs(w)
    if w.lengths is not None:
        cu = workloads.cu_seqlens(w)
        o, lse = fa2.forward_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), cu.cuda(), max(w.lengths),
                                    causal=w.causal, window=w.window)
    else:
        o, lse = fa2.forward(q.cuda(), k.cuda(), v.cuda(), causal=w.causal, n_splits=w.n_splits, window=w.window)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    if w.lengths is not None:
        # each sequence against the dense oracle on its own rows: all rows of
        # short sequences, a seeded sample (first and last included) of long ones
        g = np.random.default_rng(w.seed)
        G = w.H // w.kv_heads
        for b, (q0, q1) in enumerate(zip(cu[:-1].tolist(), cu[1:].tolist())):
            n = q1 - q0
            rows = np.arange(n) if n <= 256 else np.unique(np.r_[0, n - 1, g.choice(n, 62, replace=False)])
            kb = np.repeat(k[:, q0:q1][None].float().numpy(), G, axis=1)
            vb = np.repeat(v[:, q0:q1][None].float().numpy(), G, axis=1)
            o_ref, l_ref = oracle.attention(q[None, :, q0:q1], kb, vb, w.scale, w.causal, rows=rows,
                                            window=w.window)
            compare(o[None, :, q0 + rows], lse[None, :, q0 + rows], o_ref, l_ref, w.dtype, f"{name} sequence {b}")
        return
    rows = workloads.sample_rows(w)
    o_ref, l_ref = oracle.attention(q, k, v, w.scale, w.causal, rows=None if rows is None else rows.numpy(),
                                    window=w.window)
    if rows is not None:
        o, lse = o[:, :, rows.numpy()], lse[:, :, rows.numpy()]
    compare(o, lse, o_ref, l_ref, w.dtype, name)


# ------------------------------------------- the pages' harness shapes, ragged

# (batch, n_queries, n_keys) of the Triton test harness, run at D in {64, 128}
HARNESS = [(4, 128, 128), (2, 1024, 1024), (2, 100, 100), (1, 37, 53), (1, 200, 96)]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,M,N", HARNESS)
def test_harness_shapes(B, M, N, D, causal, dtype):
    check_case(B, 2, M, N, D, dtype, causal, seed=M + N + D)


# sizes around the 128-row query tile and the 64/32-key K/V tiles
EDGES = [(1, 1), (1, 300), (300, 1), (31, 33), (63, 65), (64, 64), (65, 63), (127, 129),
         (128, 128), (129, 127), (255, 257), (257, 255), (1000, 3000), (3000, 1000)]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("M,N", EDGES)
def test_tile_edges(M, N, causal, dtype):
    D = 128 if (M + N) % 2 else 64
    check_case(1, 3, M, N, D, dtype, causal, seed=7 * M + N)


# the shape sweep of the Triton numerics harness (causal bf16), trimmed to
# what the oracle finishes in seconds
@pytest.mark.parametrize("B,H,N,D", [(1, 8, 512, 64), (1, 8, 2048, 64), (1, 4, 4096, 128)])
def test_numerics_sweep(B, H, N, D):
    check_case(B, H, N, N, D, "bf16", True, seed=N + D)


def test_large_magnitude_scores():
    # scores with std ~16 and maxima past the fp32 exp overflow point
    check_case(2, 2, 333, 777, 64, "bf16", False, seed=11, qk_sigma=4.0)
    check_case(2, 2, 333, 777, 128, "f32", True, seed=12, qk_sigma=3.0)
    check_case(2, 2, 333, 777, 128, "f16", False, seed=13, qk_sigma=4.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_running_max_jumps_late(D, causal, dtype):
    # Keys planted deep into the sequence as 2, 8 and 16 times a late query
    # row: that row's max (scaled scores in log2 units) grows from ~4 in its
    # first tile to ~27, ~110 and ~220 long after it, the last past fp32's
    # exp range, and the other rows see scores of std up to ~28 at those
    # keys.  The running max and the rescale of O and l must follow
    # every jump, small or large.
    B, H, M, N = 1, 2, 700, 1000
    what = f"max jumps D={D} {dtype} causal={causal}"
    note("case " + what)
    q, k, v = workloads.make_inputs(B, H, M, N, D, dtype, seed=31 + D)
    target = M - 5
    for key, factor in ((150, 2.0), (420, 8.0), (690, 16.0)):
        # powers of two keep the planted keys exact in every dtype
        k[:, :, key] = q[:, :, target] * factor
    o, lse = run_gpu(q, k, v, causal)
    o_ref, l_ref = oracle.attention(q, k, v, 1.0 / math.sqrt(D), causal)
    assert l_ref[0, 0, target] > 125, "the planted key dominates the target row"
    compare(o, lse, o_ref, l_ref, dtype, what)


# ------------------------------------------------------ closed-form examples

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c["name"])
def test_golden_worked_examples(case, dtype):
    q, k, v, scale, causal, o_exp, l_exp = build_case(case)
    td = workloads.torch_dtype(dtype)
    tq, tk, tv = (torch.from_numpy(x).to(td) for x in (q, k, v))
    # the examples use values exact in bf16 and fp16, so every dtype sees the
    # same inputs
    assert torch.equal(tq.float(), torch.from_numpy(q)) and torch.equal(tv.float(), torch.from_numpy(v))
    o, lse = run_gpu(tq, tk, tv, causal, scale)
    compare(o, lse, o_exp, l_exp, dtype, case["name"] + " " + dtype)
    if dtype == "bf16" and "o_bf16_rne" in case:
        # exact tie: round-to-nearest-even is the only admissible result
        assert np.all(o == case["o_bf16_rne"]), np.unique(o)


# ---------------------------------------------------------------- properties

def test_rows_independent_of_batching():
    # each (b,h) slice gives bitwise the result it gives alone
    import exact_attention_23_amd as fa2
    q, k, v = workloads.make_inputs(2, 3, 200, 150, 128, "bf16", seed=21)
    dq, dk, dv = (t.cuda() for t in (q, k, v))
    o, lse = fa2.forward(dq, dk, dv, causal=True)
    for b, h in [(0, 0), (1, 2)]:
        o1, l1 = fa2.forward(dq[b:b + 1, h:h + 1].contiguous(), dk[b:b + 1, h:h + 1].contiguous(),
                             dv[b:b + 1, h:h + 1].contiguous(), causal=True)
        assert torch.equal(o[b, h], o1[0, 0]) and torch.equal(lse[b, h], l1[0, 0])


def test_runs_on_a_side_stream():
    import exact_attention_23_amd as fa2
    q, k, v = workloads.make_inputs(1, 4, 256, 256, 64, "f32", seed=22)
    dq, dk, dv = (t.cuda() for t in (q, k, v))
    ref_o, ref_l = fa2.forward(dq, dk, dv)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, lse = fa2.forward(dq, dk, dv)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)
