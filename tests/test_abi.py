"""Host-side tests of the C ABI (no GPU needed).

Every argument check of fa2_fwd runs before any HIP call, so invalid calls
can be exercised with fake pointers on a machine without a GPU.  Nothing
here launches a kernel.
"""
import ctypes
import os
import re
import subprocess

import pytest

import exact_attention_23_amd as fa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")

def _no_device():
    # counting devices does not initialise the GPU on this image
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:  # pragma: no cover
        return False


# calls that pass every argument check reach a kernel launch: with the fake
# pointers below they may only run where the runtime has no device to launch on
no_device_only = pytest.mark.skipif(not _no_device(), reason="would launch a kernel on fake pointers")

A = 0x10000  # fake, 16-byte aligned, non-overlapping "device" addresses
Q, K, V, O, L = A, 2 * A, 3 * A, 4 * A, 5 * A


def call(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, M=16, N=16, D=64, scale=0.125, causal=0,
         dtype=fa2.FA2_DTYPE_F32):
    return fa2.fa2_fwd(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype, None)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa2_\w+)\s*\(", text)))


def test_header_declares_exactly_the_exported_symbols():
    assert declared_functions() == sorted(fa2.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", fa2.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, f"{name} declared in fa2.h but not exported"
    lib = ctypes.CDLL(fa2.library_path())
    for name in declared_functions():
        assert hasattr(lib, name)


def test_library_is_built_for_gfx950_only(tmp_path):
    llvm = "/opt/rocm/llvm/bin"
    if not os.path.exists(os.path.join(llvm, "clang-offload-bundler")):
        pytest.skip("ROCm LLVM tools unavailable")
    fatbin = tmp_path / "fatbin.bin"
    subprocess.run([os.path.join(llvm, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fatbin}",
                    fa2.library_path(), str(tmp_path / "copy.so")], check=True)
    out = subprocess.run([os.path.join(llvm, "clang-offload-bundler"), "--list", "--type=o",
                          f"--input={fatbin}"], capture_output=True, text=True, check=True)
    targets = [t for t in out.stdout.split() if "amdgcn" in t]
    assert targets and all(t.endswith("gfx950") for t in targets), targets


def test_status_strings():
    for st in (fa2.FA2_OK, fa2.FA2_ERR_INVALID_ARGUMENT, fa2.FA2_ERR_UNSUPPORTED,
               fa2.FA2_ERR_LAUNCH, fa2.FA2_ERR_NO_DEVICE):
        s = fa2.fa2_status_string(st)
        assert s.startswith("FA2_")
    assert "unknown" in fa2.fa2_status_string(99)


@pytest.mark.parametrize("kw", [dict(q=0), dict(k=0), dict(v=0), dict(o=0), dict(lse=0)])
def test_null_pointers_rejected(kw):
    assert call(**kw) == fa2.FA2_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(B=-1), dict(H=-2), dict(M=-1), dict(N=0), dict(N=-5),
                                dict(D=0), dict(D=-64)])
def test_bad_sizes_rejected(kw):
    assert call(**kw) == fa2.FA2_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("scale", [0.0, -0.1, float("inf"), float("nan")])
def test_bad_scale_rejected(scale):
    assert call(scale=scale) == fa2.FA2_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(dtype=3), dict(dtype=-1), dict(causal=2), dict(causal=-1)])
def test_bad_enums_rejected(kw):
    assert call(**kw) == fa2.FA2_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(q=Q + 8), dict(k=K + 4), dict(v=V + 2), dict(o=O + 8), dict(lse=L + 2)])
def test_misaligned_pointers_rejected(kw):
    assert call(**kw) == fa2.FA2_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("D", [16, 32, 96, 256, 65])
def test_unsupported_head_dim(D):
    assert call(D=D) == fa2.FA2_ERR_UNSUPPORTED
    assert call(D=D, dtype=fa2.FA2_DTYPE_BF16) == fa2.FA2_ERR_UNSUPPORTED


def test_oversized_head_rejected_before_launch():
    assert call(M=1 << 25, D=64) == fa2.FA2_ERR_UNSUPPORTED
    assert call(N=1 << 25, D=128) == fa2.FA2_ERR_UNSUPPORTED


def test_overlapping_outputs_rejected():
    # o overlapping q, and lse inside o
    assert call(o=Q) == fa2.FA2_ERR_INVALID_ARGUMENT
    assert call(lse=O + 16) == fa2.FA2_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(M=0), dict(B=0), dict(H=0)])
def test_empty_problem_is_a_no_op(kw):
    # returns before touching the HIP runtime, so this is safe without a GPU
    assert call(**kw) == fa2.FA2_OK
    assert call(dtype=fa2.FA2_DTYPE_BF16, causal=1, D=128, **kw) == fa2.FA2_OK


def test_single_hip_runtime_in_process():
    # The binding must share torch's HIP runtime: pointers and streams come
    # from torch.  A second runtime copy would make every launch fail.
    import torch  # noqa: F401
    assert len(fa2._hip_runtimes_mapped()) <= 1, fa2._hip_runtimes_mapped()


# --------------------------------------------------- fa2_fwd_ex (no launches)

def call_ex(H=4, Hk=4, M=16, N=16, D=64, n_splits=1, ws=None, ws_size=0, dtype=None, causal=0):
    dtype = fa2.FA2_DTYPE_F32 if dtype is None else dtype
    return fa2.fa2_fwd_ex(Q, K, V, O, L, 1, H, Hk, M, N, D, 0.125, causal, dtype, n_splits, ws, ws_size, None)


@pytest.mark.parametrize("H,Hk", [(4, 0), (4, 3), (4, 8), (4, -1)])
def test_ex_rejects_bad_kv_head_count(H, Hk):
    assert call_ex(H=H, Hk=Hk) == fa2.FA2_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("n_splits", [-1, fa2.FA2_MAX_SPLITS + 1])
def test_ex_rejects_bad_split_count(n_splits):
    assert call_ex(n_splits=n_splits) == fa2.FA2_ERR_INVALID_ARGUMENT


def test_ex_split_needs_a_workspace():
    W = 8 * A
    need = fa2.fa2_fwd_workspace_bytes(1, 4, 16, 64, 3)
    assert call_ex(n_splits=3) == fa2.FA2_ERR_INVALID_ARGUMENT                       # none
    assert call_ex(n_splits=3, ws=W, ws_size=need - 1) == fa2.FA2_ERR_INVALID_ARGUMENT  # short
    assert call_ex(n_splits=3, ws=W + 8, ws_size=need) == fa2.FA2_ERR_INVALID_ARGUMENT  # misaligned
    assert call_ex(n_splits=3, ws=O - 64, ws_size=need) == fa2.FA2_ERR_INVALID_ARGUMENT  # overlaps o
    assert call_ex(n_splits=3, ws=W, ws_size=-5) == fa2.FA2_ERR_INVALID_ARGUMENT


def test_ex_empty_problem_needs_no_launch():
    # M == 0 with a valid split request: checks pass, nothing is enqueued
    W = 8 * A
    assert call_ex(M=0, n_splits=4, ws=W, ws_size=1 << 20) == fa2.FA2_OK
    assert call_ex(H=0, Hk=1) == fa2.FA2_OK


def test_ex_checks_kv_overlap_with_hk_sized_buffers():
    # k, v hold B*Hk*N*D elements: o placed right after a 1-head K is fine,
    # inside it is not
    kv_bytes = 1 * 1 * 16 * 64 * 4
    st = fa2.fa2_fwd_ex(Q, K, V, K + kv_bytes // 2, L, 1, 4, 1, 16, 16, 64, 0.125, 0,
                        fa2.FA2_DTYPE_F32, 1, None, 0, None)
    assert st == fa2.FA2_ERR_INVALID_ARGUMENT


def test_workspace_bytes():
    assert fa2.fa2_fwd_workspace_bytes(2, 3, 10, 64, 1) == 0
    rows = 4 * 2 * 3 * 10
    assert fa2.fa2_fwd_workspace_bytes(2, 3, 10, 64, 4) == -(-rows * 64 * 4 // 256) * 256 + rows * 4
    assert fa2.fa2_fwd_workspace_bytes(2, 3, 10, 64, 0) == -1
    assert fa2.fa2_fwd_workspace_bytes(-1, 3, 10, 64, 2) == -1
    assert fa2.fa2_fwd_workspace_bytes(1, 1, 1, 64, fa2.FA2_MAX_SPLITS + 1) == -1


def test_num_splits_heuristic():
    bf16 = fa2.FA2_DTYPE_BF16
    # a grid that already fills the GPU is never split
    assert fa2.fa2_fwd_num_splits(4, 16, 16, 4096, 4096, 128, 1, bf16) == 1
    # decode-like: one query tile per head, many keys
    s = fa2.fa2_fwd_num_splits(1, 8, 8, 1, 8192, 128, 0, bf16)
    assert 1 < s <= fa2.FA2_MAX_SPLITS and s <= (8192 // 64) // 2
    # few keys: at least two K/V tiles per split
    assert fa2.fa2_fwd_num_splits(1, 1, 1, 1, 128, 128, 0, bf16) == 1
    # grouped heads without a causal mask share workgroups: fewer, fuller
    # workgroups than one per query head
    assert fa2.fa2_fwd_num_splits(1, 32, 4, 1, 8192, 128, 0, bf16) == fa2.fa2_fwd_num_splits(1, 4, 4, 8, 8192, 128, 0, bf16)
    # arguments the entry point would reject
    assert fa2.fa2_fwd_num_splits(1, 1, 1, 1, 128, 96, 0, bf16) == 1
    assert fa2.fa2_fwd_num_splits(1, 6, 4, 1, 128, 128, 0, bf16) == 1


def test_bf16_head_addressed_by_32bit_buffer_size():
    # a 16-bit head of N*D*2 >= 2^31 bytes cannot be described by the kernels'
    # buffer resource: refused before any launch
    assert call(N=1 << 23, D=128, dtype=fa2.FA2_DTYPE_BF16) == fa2.FA2_ERR_UNSUPPORTED


@pytest.mark.parametrize("D,N", [(64, 1 << 23), (128, 1 << 22)])
def test_f32_head_addressed_by_32bit_buffer_size(D, N):
    # fp32 heads take the same buffer-resource copies with 4-byte elements:
    # the first N at which one head's K (V) reaches 2^31 bytes is refused
    # (N*D < 2^31 elements, so only the byte count catches it)
    f32 = fa2.FA2_DTYPE_F32
    assert call(N=N, D=D, dtype=f32) == fa2.FA2_ERR_UNSUPPORTED
    assert call(M=N, D=D, dtype=f32) == fa2.FA2_ERR_UNSUPPORTED
    assert fa2.fa2_fwd_ex(Q, K, V, O, L, 1, 1, 1, 16, N, D, 0.125, 0, f32, 1, None, 0, None) == fa2.FA2_ERR_UNSUPPORTED
    assert call_bwd(N=N, D=D, dtype=f32) == fa2.FA2_ERR_UNSUPPORTED
    assert call_bwd(M=N, N=16, D=D, dtype=f32) == fa2.FA2_ERR_UNSUPPORTED
    assert call_bwd_local(N=N, D=D, dtype=f32) == fa2.FA2_ERR_UNSUPPORTED
    assert call_local(N=N, D=D, dtype=f32) == fa2.FA2_ERR_UNSUPPORTED
    assert call_varlen(total_k=N, D=D, dtype=f32) == fa2.FA2_ERR_UNSUPPORTED
    assert call_bwd_varlen(total_k=N, D=D, dtype=f32) == fa2.FA2_ERR_UNSUPPORTED
    assert call_bwd_varlen(total_q=N, D=D, dtype=f32) == fa2.FA2_ERR_UNSUPPORTED


def call_noalloc(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, Hk=1, M=16, N=16, D=64, scale=0.125, causal=0,
                 dtype=fa2.FA2_DTYPE_BF16, n_splits=1):
    return fa2.fa2_fwd_ex_noalloc(q, k, v, o, lse, B, H, Hk, M, N, D, scale, causal, dtype, n_splits, None)


def test_noalloc_checks_match_fa2_fwd_ex():
    # the allocation-free entry point runs fa2_fwd_ex's argument checks
    for kw in (dict(q=0), dict(B=-1), dict(N=0), dict(H=4, Hk=3), dict(scale=0.0), dict(causal=2),
               dict(dtype=9), dict(n_splits=-1), dict(n_splits=fa2.FA2_MAX_SPLITS + 1), dict(o=Q),
               dict(k=K + 8)):
        assert call_noalloc(**kw) == fa2.FA2_ERR_INVALID_ARGUMENT, kw
    assert call_noalloc(D=96) == fa2.FA2_ERR_UNSUPPORTED
    assert call_noalloc(M=0, n_splits=8) == fa2.FA2_OK


def test_noalloc_refuses_partials_beyond_its_scratch():
    # partials of 8 splits x 64 heads x 4096 rows x 128 fp32 = 1 GiB: refused
    # before any HIP call; the same problem unsplit needs no scratch
    G = 1 << 32  # fake buffers far enough apart not to overlap at this size
    big = dict(q=G, k=2 * G, v=3 * G, o=4 * G, lse=5 * G, B=1, H=64, Hk=64, M=4096, N=4096, D=128, n_splits=8)
    need = fa2.fa2_fwd_workspace_bytes(1, 64, 4096, 128, 8)
    assert need > fa2.FA2_NOALLOC_SCRATCH_BYTES
    assert call_noalloc(**big) == fa2.FA2_ERR_SCRATCH
    assert "scratch" in fa2.fa2_status_string(fa2.FA2_ERR_SCRATCH)
    # the largest split count whose partials fit is accepted by the checks
    fits = max(s for s in range(2, fa2.FA2_MAX_SPLITS + 1)
               if fa2.fa2_fwd_workspace_bytes(1, 8, 64, 128, s) <= fa2.FA2_NOALLOC_SCRATCH_BYTES)
    assert fits == fa2.FA2_MAX_SPLITS or fa2.fa2_fwd_workspace_bytes(1, 8, 64, 128, fits + 1) > \
        fa2.FA2_NOALLOC_SCRATCH_BYTES


@no_device_only
def test_no_device_status():
    # a call that passes every check, in a process whose HIP runtime finds no
    # device: the launch is refused and reported as FA2_ERR_NO_DEVICE
    for dtype in (fa2.FA2_DTYPE_F32, fa2.FA2_DTYPE_BF16):
        assert call(dtype=dtype) == fa2.FA2_ERR_NO_DEVICE
        assert call_bwd(dtype=dtype) == fa2.FA2_ERR_NO_DEVICE
    assert call_local() == fa2.FA2_ERR_NO_DEVICE
    # the allocation-free entry point, unsplit and split (its scratch lookup)
    assert call_noalloc() == fa2.FA2_ERR_NO_DEVICE
    G = 1 << 32
    assert call_noalloc(q=G, k=2 * G, v=3 * G, o=4 * G, lse=5 * G, M=4, N=4096, D=128,
                        n_splits=4) == fa2.FA2_ERR_NO_DEVICE


# ------------------------------------------------------ fa2_bwd (no launches)

DO, DQ, DK, DV, DL = 6 * A, 7 * A, 8 * A, 9 * A, 10 * A


def call_bwd(q=Q, k=K, v=V, o=O, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, delta=DL, B=1, H=2, Hk=2, M=16,
             N=16, D=64, scale=0.125, causal=0, dtype=None):
    dtype = fa2.FA2_DTYPE_BF16 if dtype is None else dtype
    return fa2.fa2_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, Hk, M, N, D, scale, causal, dtype, None)


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "delta"])
def test_bwd_null_pointers_rejected(name):
    assert call_bwd(**{name: 0}) == fa2.FA2_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(B=-1), dict(H=-1), dict(Hk=0), dict(H=4, Hk=3), dict(M=-1), dict(N=0),
                                dict(D=0), dict(scale=0.0), dict(scale=float("nan")), dict(causal=2),
                                dict(dtype=7)])
def test_bwd_bad_arguments_rejected(kw):
    assert call_bwd(**kw) == fa2.FA2_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("name,off", [("q", 8), ("dout", 8), ("dq", 2), ("dk", 8), ("dv", 4), ("lse", 2),
                                      ("delta", 2)])
def test_bwd_misaligned_pointers_rejected(name, off):
    base = {"q": Q, "dout": DO, "dq": DQ, "dk": DK, "dv": DV, "lse": L, "delta": DL}[name]
    kw = {("do" if name == "dout" else name): base + off}
    assert call_bwd(**kw) == fa2.FA2_ERR_INVALID_ARGUMENT


def test_bwd_unsupported_head_dim_and_sizes():
    for dtype in (fa2.FA2_DTYPE_BF16, fa2.FA2_DTYPE_F16, fa2.FA2_DTYPE_F32):
        for D in (32, 96, 256):
            assert call_bwd(D=D, dtype=dtype) == fa2.FA2_ERR_UNSUPPORTED
    # the 16-bit kernels address one head's K (V) through a 32-bit byte range
    assert call_bwd(N=1 << 23, D=128) == fa2.FA2_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(dq=Q), dict(dk=V), dict(dv=DK), dict(delta=DQ + 16), dict(dq=DO),
                                dict(delta=L), dict(dk=DV + 64)])
def test_bwd_overlapping_outputs_rejected(kw):
    assert call_bwd(**kw) == fa2.FA2_ERR_INVALID_ARGUMENT


def test_bwd_empty_kv_is_a_no_op():
    # no K/V rows to write: returns before any HIP call
    assert call_bwd(B=0) == fa2.FA2_OK


def test_null_pointers_allowed_for_empty_buffers():
    # empty q/o/lse (M == 0) may be null; k/v are not empty, so not null
    assert call(q=0, o=0, lse=0, M=0) == fa2.FA2_OK
    assert call(k=0, M=0) == fa2.FA2_ERR_INVALID_ARGUMENT
    assert call_bwd(dk=0, M=0) == fa2.FA2_ERR_INVALID_ARGUMENT


@no_device_only
def test_bwd_null_query_buffers_allowed_when_empty():
    # M == 0 still writes dK = dV = 0, so the checks pass and the call reaches
    # its launch
    assert call_bwd(q=0, o=0, lse=0, do=0, dq=0, delta=0, M=0) == fa2.FA2_ERR_NO_DEVICE


# ------------------------------------------- fa2_fwd_local / fa2_fwd_varlen (no launches)

def call_local(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Hk=2, M=16, N=16, D=64, causal=0, wl=4, wr=4, dtype=None):
    dtype = fa2.FA2_DTYPE_BF16 if dtype is None else dtype
    return fa2.fa2_fwd_local(q, k, v, o, lse, B, H, Hk, M, N, D, 0.125, causal, wl, wr, dtype, None)


CQ, CK = 11 * A, 12 * A


def call_varlen(q=Q, k=K, v=V, o=O, lse=L, cq=CQ, ck=CK, B=2, H=2, Hk=2, total_q=16, total_k=16, max_q=8,
                D=64, causal=0, wl=-1, wr=-1, dtype=None):
    dtype = fa2.FA2_DTYPE_BF16 if dtype is None else dtype
    return fa2.fa2_fwd_varlen(q, k, v, o, lse, cq, ck, B, H, Hk, total_q, total_k, max_q, D, 0.125, causal,
                              wl, wr, dtype, None)


@pytest.mark.parametrize("kw", [dict(wl=-2), dict(wr=-5), dict(q=0), dict(k=0), dict(N=0), dict(Hk=3),
                                dict(causal=2), dict(o=Q), dict(lse=O + 4), dict(q=Q + 8)])
def test_local_bad_arguments_rejected(kw):
    assert call_local(**kw) == fa2.FA2_ERR_INVALID_ARGUMENT


def test_local_unsupported_and_empty():
    assert call_local(D=96) == fa2.FA2_ERR_UNSUPPORTED
    assert call_local(M=0) == fa2.FA2_OK
    assert call_local(B=0) == fa2.FA2_OK


@pytest.mark.parametrize("kw", [dict(cq=0), dict(ck=0), dict(cq=CQ + 2), dict(max_q=17), dict(max_q=-1),
                                dict(total_k=-1), dict(wl=-3), dict(q=0), dict(o=K), dict(H=4, Hk=3)])
def test_varlen_bad_arguments_rejected(kw):
    assert call_varlen(**kw) == fa2.FA2_ERR_INVALID_ARGUMENT


def test_varlen_unsupported_and_empty():
    assert call_varlen(D=32) == fa2.FA2_ERR_UNSUPPORTED
    # nothing to launch: no sequences, no heads, or no query rows anywhere
    assert call_varlen(B=0, cq=0, ck=0) == fa2.FA2_OK
    assert call_varlen(H=0) == fa2.FA2_OK
    assert call_varlen(max_q=0) == fa2.FA2_OK


# ------------------------------------------- fa2_bwd_local / fa2_bwd_varlen (no launches)

def call_bwd_local(wl=4, wr=4, **kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, delta=DL, B=1, H=2, Hk=2, M=16, N=16, D=64,
                scale=0.125, causal=0, dtype=fa2.FA2_DTYPE_BF16)
    args.update(kw)
    a = args
    return fa2.fa2_bwd_local(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["delta"],
                             a["B"], a["H"], a["Hk"], a["M"], a["N"], a["D"], a["scale"], a["causal"], wl, wr,
                             a["dtype"], None)


def call_bwd_varlen(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, delta=DL, cq=CQ, ck=CK, B=2, H=2, Hk=2,
             total_q=16, total_k=16, max_q=8, max_k=8, D=64, causal=0, wl=-1, wr=-1, dtype=fa2.FA2_DTYPE_BF16)
    a.update(kw)
    return fa2.fa2_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                              a["delta"], a["cq"], a["ck"], a["B"], a["H"], a["Hk"], a["total_q"], a["total_k"],
                              a["max_q"], a["max_k"], a["D"], 0.125, a["causal"], a["wl"], a["wr"], a["dtype"], None)


@pytest.mark.parametrize("kw", [dict(wl=-2), dict(wr=-3), dict(dq=0), dict(dk=Q), dict(N=0), dict(causal=3)])
def test_bwd_local_bad_arguments_rejected(kw):
    assert call_bwd_local(**kw) == fa2.FA2_ERR_INVALID_ARGUMENT


def test_bwd_local_unsupported():
    assert call_bwd_local(D=96) == fa2.FA2_ERR_UNSUPPORTED
    assert call_bwd_local(D=96, dtype=fa2.FA2_DTYPE_F32) == fa2.FA2_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(cq=0), dict(ck=CK + 1), dict(max_q=17), dict(max_k=-1), dict(total_q=-1),
                                dict(wl=-2), dict(dv=0), dict(delta=Q), dict(H=4, Hk=3)])
def test_bwd_varlen_bad_arguments_rejected(kw):
    assert call_bwd_varlen(**kw) == fa2.FA2_ERR_INVALID_ARGUMENT


def test_bwd_varlen_unsupported_and_empty():
    assert call_bwd_varlen(D=96, dtype=fa2.FA2_DTYPE_F32) == fa2.FA2_ERR_UNSUPPORTED
    assert call_bwd_varlen(B=0, cq=0, ck=0) == fa2.FA2_OK
