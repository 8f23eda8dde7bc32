"""Memory-safety and determinism guards for the HIP path.

* Outputs are written into the middle of larger buffers whose head and tail
  hold a sentinel pattern; the kernels must write exactly [B,H,M,D] of o and
  [B,H,M] of lse and nothing else (stores past M rows would hit the tail).
* Inputs carry NaN just past their end and just before their start: a read of
  a padded key or query row outside the tensor would poison the output.
* Three runs of one call are bitwise identical (no races, no atomics).
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_23_amd as fa2
import workloads

pytestmark = pytest.mark.gpu

PAD = 4096  # elements of canary before and after each buffer (16-byte multiple)


def padded(t, fill):
    flat = torch.full((PAD + t.numel() + PAD,), fill, dtype=t.dtype, device="cuda")
    flat[PAD:PAD + t.numel()].copy_(t.reshape(-1))
    return flat, flat[PAD:PAD + t.numel()].view(t.shape)


def call(q, k, v, o, lse, causal, dtype_code):
    B, H, M, D = q.shape
    N = k.shape[2]
    st = fa2.fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     B, H, M, N, D, 1.0 / math.sqrt(D), int(causal), dtype_code,
                     torch.cuda.current_stream().cuda_stream)
    print(f"fa2_fwd status {st}", flush=True)
    assert st == fa2.FA2_OK, fa2.fa2_status_string(st)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("M,N,D", [(1, 1, 64), (100, 37, 128), (129, 200, 64), (1000, 3000, 64), (300, 300, 128)])
def test_no_out_of_bounds_access(M, N, D, causal, dtype):
    B, H = 2, 3
    q, k, v = workloads.make_inputs(B, H, M, N, D, dtype, seed=M + N)
    code = {"f32": fa2.FA2_DTYPE_F32, "bf16": fa2.FA2_DTYPE_BF16, "f16": fa2.FA2_DTYPE_F16}[dtype]
    nan = float("nan")
    qf, dq = padded(q.cuda(), nan)
    kf, dk = padded(k.cuda(), nan)
    vf, dv = padded(v.cuda(), nan)
    sentinel = -12288.0  # exact in bf16, fp16 and fp32
    of, do = padded(torch.empty_like(q, device="cuda"), sentinel)
    lf, dl = padded(torch.empty((B, H, M), dtype=torch.float32, device="cuda"), sentinel)
    print(f"case B={B} H={H} M={M} N={N} D={D} {dtype} causal={causal}", flush=True)
    call(dq, dk, dv, do, dl, causal, code)
    torch.cuda.synchronize()
    problems = []
    for name, flat, n in (("o", of, do.numel()), ("lse", lf, dl.numel())):
        head, tail = flat[:PAD].float().cpu(), flat[PAD + n:].float().cpu()
        bad = int((head != sentinel).sum()) + int((tail != sentinel).sum())
        if bad:
            problems.append(f"{name}: {bad} canary elements overwritten")
    o_h, l_h = do.float().cpu(), dl.cpu()
    if not torch.isfinite(o_h).all():
        problems.append(f"o: {int((~torch.isfinite(o_h)).sum())} non-finite (an input read out of bounds?)")
    if not torch.isfinite(l_h).all():
        problems.append(f"lse: {int((~torch.isfinite(l_h)).sum())} non-finite")
    if torch.any(o_h == sentinel):
        problems.append(f"o: {int((o_h == sentinel).sum())} elements not written")
    if torch.any(l_h == sentinel):
        problems.append(f"lse: {int((l_h == sentinel).sum())} elements not written")
    print("problems:", problems, flush=True)
    assert not problems, "; ".join(problems)


@pytest.mark.parametrize("name", ["causal_bf16_4k", "mha_f32_2k", "ragged_bf16_cross"])
def test_bitwise_deterministic(name):
    w = workloads.get(name)
    q, k, v = (t.cuda() for t in workloads.workload_inputs(w))
    outs = [fa2.forward(q, k, v, causal=w.causal) for _ in range(3)]
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


def test_invalid_call_leaves_outputs_untouched():
    q, k, v = (t.cuda() for t in workloads.make_inputs(1, 1, 64, 64, 64, "f32", seed=3))
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 1, 64), 7.0, device="cuda")
    st = fa2.fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     1, 1, 64, 64, 96, 0.1, 0, fa2.FA2_DTYPE_F32, None)
    assert st == fa2.FA2_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)


def test_wrong_output_buffers_refused_before_launch():
    # caller-supplied outputs that are short, mistyped, strided or absent from
    # the device raise before any launch, and the buffers keep their contents
    q, k, v = (t.cuda() for t in workloads.make_inputs(1, 2, 64, 64, 64, "bf16", seed=5))
    bad_outs = [torch.full((1, 2, 63, 64), 7.0, dtype=torch.bfloat16, device="cuda"),
                torch.full((1, 2, 64, 64), 7.0, dtype=torch.float32, device="cuda"),
                torch.full((1, 2, 64, 128), 7.0, dtype=torch.bfloat16, device="cuda")[..., :64],
                torch.full((1, 2, 64, 64), 7.0, dtype=torch.bfloat16)]
    for out in bad_outs:
        with pytest.raises(ValueError):
            fa2.forward(q, k, v, out=out)
    for lse in (torch.full((1, 2, 63), 7.0, device="cuda"),
                torch.full((1, 2, 64), 7.0, dtype=torch.float64, device="cuda")):
        with pytest.raises(ValueError):
            fa2.forward(q, k, v, lse=lse)
    # packed sequences: [H, total, D] with two sequences of 40 and 24 rows
    qp, kp, vp = (t.reshape(2, 64, 64).contiguous() for t in (q, k, v))
    cu = torch.tensor([0, 40, 64], dtype=torch.int32, device="cuda")
    short = torch.full((2, 60, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fa2.forward_varlen(qp, kp, vp, cu, cu, 40, out=short)
    with pytest.raises(ValueError):
        fa2.forward_varlen(qp, kp, vp, cu, cu, 40, lse=torch.full((2, 64), 7.0, dtype=torch.bfloat16,
                                                                     device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(short == 7.0) and all(torch.all(o == 7.0) for o in bad_outs)
