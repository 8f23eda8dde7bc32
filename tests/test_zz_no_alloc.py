"""fa2_fwd_ex_noalloc, the entry point for callers that cannot allocate: the
split-K/V partials live in the library's static device scratch array.

Called through the C ABI with raw device pointers, its output must equal
fa2_fwd_ex's (same kernels, same split partition: bitwise) and the oracle's
to the parity tolerances, on two calls in a row, the second with a smaller
problem (the array keeps the first call's partials; nothing in it may leak
into the second result).
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

CODES = {"f32": fa2.FA2_DTYPE_F32, "bf16": fa2.FA2_DTYPE_BF16, "f16": fa2.FA2_DTYPE_F16}


def run_pair(B, H, Hk, M, N, D, dtype, causal, n_splits, seed):
    """(noalloc o, lse), (fa2_fwd_ex o, lse), the effective split count."""
    q, k, v = workloads.make_inputs(B, H, M, N, D, dtype, seed, Hk=Hk)
    dq, dk, dv = (t.to("cuda") for t in (q, k, v))
    code = CODES[dtype]
    splits = fa2.fa2_fwd_num_splits(B, H, Hk, M, N, D, int(causal), code) if n_splits == 0 else n_splits
    stream = torch.cuda.current_stream().cuda_stream
    scale = 1.0 / math.sqrt(D)
    o1 = torch.full_like(dq, 7.0)
    l1 = torch.full((B, H, M), 7.0, dtype=torch.float32, device="cuda")
    st = fa2.fa2_fwd_ex_noalloc(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), o1.data_ptr(), l1.data_ptr(),
                                B, H, Hk, M, N, D, scale, int(causal), code, n_splits, stream)
    assert st == fa2.FA2_OK, fa2.fa2_status_string(st)
    o2 = torch.empty_like(dq)
    l2 = torch.empty((B, H, M), dtype=torch.float32, device="cuda")
    need = fa2.fa2_fwd_workspace_bytes(B, H, M, D, splits)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    st = fa2.fa2_fwd_ex(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                        B, H, Hk, M, N, D, scale, int(causal), code, n_splits, ws.data_ptr(), ws.numel(), stream)
    assert st == fa2.FA2_OK, fa2.fa2_status_string(st)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, scale, causal)
    return (o1, l1), (o2, l2), (o_ref, l_ref), splits


@pytest.mark.parametrize("first,second", [
    # (B, H, Hk, M, N, D, dtype, causal, n_splits): a decode-like call with the
    # library's split count, then a smaller one with fewer splits
    ((2, 8, 2, 4, 3000, 128, "bf16", False, 0), (1, 4, 1, 1, 1000, 64, "f16", False, 4)),
    ((1, 4, 4, 300, 2000, 64, "f32", True, 8), (1, 2, 2, 70, 200, 64, "f32", True, 3)),
    # the second call unsplit: no scratch at all
    ((1, 8, 8, 16, 4096, 128, "bf16", True, 16), (1, 1, 1, 33, 129, 128, "bf16", False, 1)),
])
def test_noalloc_matches_fa2_fwd_ex(first, second):
    for i, case in enumerate((first, second)):
        B, H, Hk, M, N, D, dtype, causal, n_splits = case
        what = f"call {i + 1}: B={B} H={H} Hk={Hk} M={M} N={N} D={D} {dtype} causal={causal} splits={n_splits}"
        note("case " + what)
        (o1, l1), (o2, l2), (o_ref, l_ref), splits = run_pair(B, H, Hk, M, N, D, dtype, causal, n_splits,
                                                              seed=i + M + N)
        note(f"  effective splits {splits}")
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{what}: differs from fa2_fwd_ex"
        compare(o1.float().cpu().numpy().astype(np.float64), l1.cpu().numpy().astype(np.float64),
                o_ref, l_ref, dtype, what)


def test_noalloc_refuses_oversized_partials_without_touching_outputs():
    B, H, M, N, D = 1, 64, 512, 4096, 128
    assert fa2.fa2_fwd_workspace_bytes(B, H, M, D, 8) > fa2.FA2_NOALLOC_SCRATCH_BYTES
    q, k, v = (torch.zeros((B, H, n, D), dtype=torch.bfloat16, device="cuda") for n in (M, N, N))
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, H, M), 7.0, device="cuda")
    st = fa2.fa2_fwd_ex_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                B, H, H, M, N, D, 0.088, 0, fa2.FA2_DTYPE_BF16, 8,
                                torch.cuda.current_stream().cuda_stream)
    assert st == fa2.FA2_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)
