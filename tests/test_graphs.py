"""The entry points inside a captured HIP graph.

fa2_fwd_ex (split K/V and its combine kernel included) and fa2_bwd launch
kernels only on the caller's stream -- no allocation, no host
synchronisation, no memset -- so a serving loop can capture them once and
replay the graph.  Each test captures with static input tensors, then for
several fresh inputs copies them in, replays, and checks the replay against
an eager call on the same inputs: bitwise, since the kernels are the same
and deterministic.  Eager work and synchronisations run between the replays.
"""
import pytest
import torch

import exact_attention_23_amd as fa2
import workloads
from tests.test_parity import note

pytestmark = pytest.mark.gpu


def _capture(fn):
    # warm up on a side stream (default priority), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = fn()
    torch.cuda.synchronize()
    return graph, outs


def test_decode_split_forward_replays_in_a_graph():
    # few query rows over many keys: split K/V plus the combine kernel
    B, H, Hk, M, N, D = 2, 8, 2, 4, 3000, 128
    code = fa2.FA2_DTYPE_BF16
    splits = fa2.fa2_fwd_num_splits(B, H, Hk, M, N, D, 0, code)
    assert splits > 1
    note(f"graph decode forward, {splits} splits")
    q, k, v = (t.cuda() for t in workloads.make_inputs(B, H, M, N, D, "bf16", 1, Hk=Hk))
    ws = torch.empty(fa2.fa2_fwd_workspace_bytes(B, H, M, D, splits), dtype=torch.uint8, device="cuda")
    graph, (o, lse) = _capture(lambda: fa2.forward(q, k, v, n_splits=splits, workspace=ws))
    for seed in (2, 3, 4):
        nq, nk, nv = (t.cuda() for t in workloads.make_inputs(B, H, M, N, D, "bf16", seed, Hk=Hk))
        q.copy_(nq), k.copy_(nk), v.copy_(nv)
        graph.replay()
        torch.cuda.synchronize()
        o_ref, l_ref = fa2.forward(nq, nk, nv, n_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"replay with seed {seed}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causal_forward_backward_replays_in_a_graph(dtype):
    B, H, M, N, D = 1, 4, 300, 300, 64
    note(f"graph forward + backward, {dtype}")
    q, k, v = (t.cuda() for t in workloads.make_inputs(B, H, M, N, D, dtype, 5))
    do = workloads.make_dout(B, H, M, D, dtype, 5).cuda()

    def step():
        o, lse = fa2.forward(q, k, v, causal=True)
        return (o, lse) + fa2.backward(q, k, v, o, lse, do, causal=True)

    graph, outs = _capture(step)
    for seed in (6, 7, 8):
        nq, nk, nv = (t.cuda() for t in workloads.make_inputs(B, H, M, N, D, dtype, seed))
        ndo = workloads.make_dout(B, H, M, D, dtype, seed).cuda()
        q.copy_(nq), k.copy_(nk), v.copy_(nv), do.copy_(ndo)
        graph.replay()
        torch.cuda.synchronize()
        o, lse = fa2.forward(nq, nk, nv, causal=True)
        ref = (o, lse) + fa2.backward(nq, nk, nv, o, lse, ndo, causal=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), outs, ref):
            assert torch.equal(a, b), f"{name} differs on the replay with seed {seed}"
