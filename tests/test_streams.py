"""Calls on several HIP streams at once.

The library keeps no state between calls and every entry point only
enqueues kernels on the stream it is given, so independent calls on
different streams may run concurrently.  Two streams (default priority)
each queue forwards (one of them split K/V) and a backward on their own
inputs; the results must equal the same calls made one after another
(bitwise: same kernels, deterministic).
"""
import pytest
import torch

import exact_attention_23_amd as fa2
import workloads
from tests.test_parity import note

pytestmark = pytest.mark.gpu


def _work(q, k, v, do, splits):
    o, lse = fa2.forward(q, k, v, causal=True)
    o2, l2 = fa2.forward(q[:, :, :8].contiguous(), k, v, n_splits=splits)
    grads = fa2.backward(q, k, v, o, lse, do, causal=True)
    return (o, lse, o2, l2) + grads


def test_two_streams_match_sequential_calls():
    note("case two streams, bf16, causal forward + split forward + backward")
    data = []
    for seed in (1, 2):
        q, k, v = (t.cuda() for t in workloads.make_inputs(2, 8, 700, 700, 128, "bf16", seed, Hk=2))
        do = workloads.make_dout(2, 8, 700, 128, "bf16", seed).cuda()
        data.append((q, k, v, do))
    ref = [_work(*d, splits=4) for d in data]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    for rep in range(3):
        for i, (s, d) in enumerate(zip(streams, data)):
            with torch.cuda.stream(s):
                outs[i] = _work(*d, splits=4)
    torch.cuda.synchronize()
    for i in range(2):
        for name, a, b in zip(("o", "lse", "o_split", "lse_split", "dq", "dk", "dv"), outs[i], ref[i]):
            assert torch.equal(a, b), f"stream {i}: {name} differs from the sequential call"
