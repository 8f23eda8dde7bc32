"""Grouped-query heads and split K/V through fa2_fwd_ex, against the oracle.

Tolerances are those of the unsplit path (fp32: 1e-4 on O and L; bf16: 2e-2
on O, 1e-3 on L).  Split K/V re-associates the softmax sums (per-range
partials combined through their logsumexp), so it is compared with the
oracle, and with the unsplit kernel only to within the same tolerances.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_23_amd as fa2
import oracle
import workloads
from tests.test_parity import compare, note

pytestmark = pytest.mark.gpu


def run(q, k, v, causal, n_splits=1, workspace=None):
    dq, dk, dv = (t.to("cuda") for t in (q, k, v))
    o, lse = fa2.forward(dq, dk, dv, causal=causal, n_splits=n_splits, workspace=workspace)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(B, H, Hk, M, N, D, dtype, causal, n_splits=1, seed=0, qk_sigma=1.0):
    what = f"B={B} H={H} Hk={Hk} M={M} N={N} D={D} {dtype} causal={causal} splits={n_splits}"
    note("case " + what)
    q, k, v = workloads.make_inputs(B, H, M, N, D, dtype, seed, qk_sigma, Hk=Hk)
    o, lse = run(q, k, v, causal, n_splits)
    o_ref, l_ref = oracle.attention(q, k, v, 1.0 / math.sqrt(D), causal)
    return compare(o, lse, o_ref, l_ref, dtype, what)


# ------------------------------------------------------------ grouped query

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H,Hk", [(8, 1), (8, 2), (6, 3)])
@pytest.mark.parametrize("M,N", [(300, 300), (100, 517), (513, 64)])
def test_grouped_query_heads(M, N, H, Hk, D, causal, dtype):
    check(2, H, Hk, M, N, D, dtype, causal, seed=M + N + Hk)


def test_gqa_equals_mha_on_repeated_heads():
    # every query head reading its group's K/V head == MHA with the K/V heads
    # repeated: same kernel arithmetic, so bitwise equal
    q, k, v = workloads.make_inputs(2, 8, 333, 401, 128, "bf16", 5, Hk=2)
    o1, l1 = run(q, k, v, True)
    o2, l2 = run(q, k.repeat_interleave(4, dim=1).contiguous(), v.repeat_interleave(4, dim=1).contiguous(), True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------- split K/V

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n_splits", [2, 3, 8])
def test_split_kv(n_splits, D, causal, dtype):
    check(1, 4, 4, 300, 1000, D, dtype, causal, n_splits=n_splits, seed=n_splits)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_split_kv_more_splits_than_tiles(causal, dtype):
    # 50 splits over N = 200 keys: most ranges are empty (L = -inf partials)
    check(1, 2, 2, 70, 200, 64, dtype, causal, n_splits=50, seed=11)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("M", [1, 4, 37])
def test_split_kv_decode_shapes_auto(M, dtype):
    # few query rows over many keys: the case split K/V exists for
    B, H, N, D = 2, 8, 4096, 128
    code = {"f32": fa2.FA2_DTYPE_F32, "bf16": fa2.FA2_DTYPE_BF16, "f16": fa2.FA2_DTYPE_F16}[dtype]
    splits = fa2.fa2_fwd_num_splits(B, H, 2, M, N, D, 0, code)
    note(f"auto splits for M={M}: {splits}")
    assert splits > 1
    check(B, H, 2, M, N, D, dtype, False, n_splits=0, seed=M)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("M,N,H,Hk,n_splits", [
    (1, 3000, 8, 1, 0),      # one token per query head, 8 heads on one K/V head
    (16, 777, 8, 2, 1),      # 64 grouped rows, unsplit, ragged N
    (8, 5000, 32, 4, 0),     # 64 grouped rows, automatic splits
    (33, 129, 4, 4, 3),      # explicit splits over a short key range
    (64, 1000, 2, 2, 0),     # the largest row count of the few-row kernels
    (65, 1000, 2, 2, 0),     # one row more: the 256-row kernels
    (16, 4500, 8, 2, 3),     # splits of 1500 keys (D = 128, 16-bit, no mask: the four-buffer ring),
                             # 47 tiles of 32 keys per split, the last one ragged
    (4, 9000, 4, 4, 2),      # splits of 4500 keys: 141 tiles per split, one past a multiple of four
])
def test_few_query_rows(M, N, H, Hk, n_splits, causal, D, dtype):
    # rows per (K/V) head <= 64 run the 64-row workgroups; the result must not
    # depend on which kernel served it beyond the tolerances
    check(2, H, Hk, M, N, D, dtype, causal, n_splits=n_splits, seed=M * 7 + N)


def test_split_kv_large_magnitude():
    # scores far beyond fp32 exp range in every split (the workload with
    # qk_sigma = 4): the merge must rescale by logsumexp differences only
    check(2, 4, 4, 200, 3000, 64, "bf16", False, n_splits=6, seed=3, qk_sigma=4.0)


def test_split_kv_deterministic_and_close_to_unsplit():
    q, k, v = workloads.make_inputs(1, 8, 256, 2048, 128, "bf16", 9)
    runs = [run(q, k, v, True, n_splits=4) for _ in range(2)]
    assert np.array_equal(runs[0][0], runs[1][0]) and np.array_equal(runs[0][1], runs[1][1])
    o1, l1 = run(q, k, v, True, n_splits=1)
    assert np.abs(runs[0][0] - o1).max() <= 2e-2 and np.abs(runs[0][1] - l1).max() <= 1e-3


def test_split_kv_writes_only_o_and_lse():
    # canaries around o, lse and the workspace: nothing outside is written
    B, H, M, N, D = 1, 3, 90, 700, 64
    q, k, v = (t.cuda() for t in workloads.make_inputs(B, H, M, N, D, "bf16", 4))
    PAD = 4096
    splits = 5
    need = fa2.fa2_fwd_workspace_bytes(B, H, M, D, splits)
    o_buf = torch.full((PAD + B * H * M * D + PAD,), -12288.0, dtype=torch.bfloat16, device="cuda")
    l_buf = torch.full((PAD + B * H * M + PAD,), -12288.0, dtype=torch.float32, device="cuda")
    w_buf = torch.full((PAD + need // 4 + PAD,), -12288.0, dtype=torch.float32, device="cuda")
    o = o_buf[PAD:PAD + B * H * M * D]
    lse = l_buf[PAD:PAD + B * H * M]
    ws = w_buf[PAD:PAD + need // 4]
    st = fa2.fa2_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        B, H, H, M, N, D, 1 / math.sqrt(D), 1, fa2.FA2_DTYPE_BF16, splits,
                        ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert st == fa2.FA2_OK, fa2.fa2_status_string(st)
    torch.cuda.synchronize()
    for name, buf, n in (("o", o_buf, o.numel()), ("lse", l_buf, lse.numel()), ("workspace", w_buf, ws.numel())):
        head, tail = buf[:PAD].float().cpu(), buf[PAD + n:].float().cpu()
        assert bool((head == -12288.0).all()) and bool((tail == -12288.0).all()), f"{name} canary overwritten"
    o_ref, l_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), 1 / math.sqrt(D), True)
    compare(o.view(B, H, M, D).float().cpu().numpy(), lse.view(B, H, M).cpu().numpy(), o_ref, l_ref, "bf16",
            "canary split case")


def test_short_workspace_is_rejected_before_launch():
    q, k, v = (t.cuda() for t in workloads.make_inputs(1, 2, 64, 512, 64, "f32", 1))
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 2, 64), 7.0, device="cuda")
    need = fa2.fa2_fwd_workspace_bytes(1, 2, 64, 64, 4)
    ws = torch.empty(need - 4, dtype=torch.uint8, device="cuda")
    st = fa2.fa2_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        1, 2, 2, 64, 512, 64, 0.125, 0, fa2.FA2_DTYPE_F32, 4, ws.data_ptr(), need - 4, None)
    assert st == fa2.FA2_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
