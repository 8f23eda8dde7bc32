"""Python binding of libfa2 (exact attention forward and backward passes on gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfa2.so``.  PyTorch is used for device memory and streams.
There is no CPU fallback: if the library is missing, importing the binding
raises.

``fa2_fwd``, ``fa2_fwd_ex``, ``fa2_fwd_ex_noalloc``, ``fa2_fwd_workspace_bytes``,
``fa2_fwd_num_splits``, ``fa2_fwd_local``, ``fa2_fwd_varlen``, ``fa2_bwd``,
``fa2_bwd_local`` and ``fa2_bwd_varlen`` mirror the C entry points of
``include/fa2.h`` one to one (raw device pointers and sizes).  ``forward``,
``forward_varlen``, ``backward`` and ``backward_varlen`` are the tensor-level
conveniences that allocate outputs (and any split-K/V workspace) with torch
and call the library on the current stream;
``attention`` wraps forward and backward in a ``torch.autograd.Function``.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["FA2_DTYPE_F32", "FA2_DTYPE_BF16", "FA2_DTYPE_F16", "FA2_OK", "FA2_ERR_INVALID_ARGUMENT",
           "FA2_ERR_UNSUPPORTED", "FA2_ERR_LAUNCH", "FA2_ERR_NO_DEVICE", "FA2_ERR_SCRATCH", "FA2_MAX_SPLITS",
           "FA2_NOALLOC_SCRATCH_BYTES", "Fa2Error", "fa2_fwd", "fa2_fwd_ex", "fa2_fwd_ex_noalloc", "fa2_fwd_workspace_bytes", "fa2_fwd_num_splits", "fa2_fwd_local",
           "fa2_fwd_varlen", "fa2_bwd", "fa2_bwd_local", "fa2_bwd_varlen", "fa2_status_string", "forward",
           "forward_varlen", "backward", "backward_varlen", "attention", "library_path", "EXPORTED_SYMBOLS"]

FA2_DTYPE_F32 = 0
FA2_DTYPE_BF16 = 1
FA2_DTYPE_F16 = 2

FA2_OK = 0
FA2_ERR_INVALID_ARGUMENT = 1
FA2_ERR_UNSUPPORTED = 2
FA2_ERR_LAUNCH = 3
FA2_ERR_NO_DEVICE = 4
FA2_ERR_SCRATCH = 5

FA2_MAX_SPLITS = 128
FA2_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024

EXPORTED_SYMBOLS = ("fa2_bwd", "fa2_bwd_local", "fa2_bwd_varlen", "fa2_fwd", "fa2_fwd_ex", "fa2_fwd_ex_noalloc",
                    "fa2_fwd_local",
                    "fa2_fwd_num_splits", "fa2_fwd_varlen", "fa2_fwd_workspace_bytes", "fa2_status_string")

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfa2.so")


def library_path() -> str:
    return _LIB_PATH


def _hip_runtimes_mapped():
    """Distinct HIP runtime library files mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                parts = line.split()
                if len(parts) >= 6 and "libamdhip64" in parts[-1]:
                    paths.add(os.path.realpath(parts[-1]))
    except OSError:
        pass
    return paths


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python exact_attention_23_amd/build.py` "
            "(there is no fallback implementation)")
    # Device memory and streams come from torch, so libfa2 must bind to torch's
    # HIP runtime.  Importing torch first makes the loader resolve libfa2's
    # libamdhip64.so.7 dependency to the copy torch already mapped; loading
    # libfa2 first would map a second, different HIP runtime into the process.
    import torch  # noqa: F401
    lib = ctypes.CDLL(_LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError("two different HIP runtimes are loaded in this process "
                          f"({sorted(runtimes)}); import torch before loading libfa2")
    lib.fa2_fwd.restype = ctypes.c_int
    lib.fa2_fwd.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
    ]
    lib.fa2_fwd_ex.restype = ctypes.c_int
    lib.fa2_fwd_ex.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
    ]
    lib.fa2_fwd_ex_noalloc.restype = ctypes.c_int
    lib.fa2_fwd_ex_noalloc.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
    ]
    lib.fa2_fwd_workspace_bytes.restype = ctypes.c_int64
    lib.fa2_fwd_workspace_bytes.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int]
    lib.fa2_fwd_num_splits.restype = ctypes.c_int
    lib.fa2_fwd_num_splits.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int, ctypes.c_int]
    lib.fa2_fwd_local.restype = ctypes.c_int
    lib.fa2_fwd_local.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.fa2_fwd_varlen.restype = ctypes.c_int
    lib.fa2_fwd_varlen.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 7 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.fa2_bwd.restype = ctypes.c_int
    lib.fa2_bwd.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa2_bwd_local.restype = ctypes.c_int
    lib.fa2_bwd_local.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.fa2_bwd_varlen.restype = ctypes.c_int
    lib.fa2_bwd_varlen.argtypes = [ctypes.c_void_p] * 12 + [ctypes.c_int64] * 8 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.fa2_status_string.restype = ctypes.c_char_p
    lib.fa2_status_string.argtypes = [ctypes.c_int]
    return lib


_lib = _load()


class Fa2Error(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(fa2_status_string(status))


def fa2_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, M: int, N: int, D: int,
            scale: float, causal: int, dtype: int, stream: int | None) -> int:
    """Direct call of the C entry point; pointers are integers (device
    addresses).  Returns the fa2_status code."""
    return int(_lib.fa2_fwd(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype, stream))


def fa2_fwd_ex(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Hk: int, M: int, N: int,
               D: int, scale: float, causal: int, dtype: int, n_splits: int, workspace: int | None,
               workspace_size: int, stream: int | None) -> int:
    """Direct call of the extended C entry point (grouped-query heads, split
    K/V); pointers are integers.  Returns the fa2_status code."""
    return int(_lib.fa2_fwd_ex(q, k, v, o, lse, B, H, Hk, M, N, D, scale, causal, dtype, n_splits,
                               workspace, workspace_size, stream))


def fa2_fwd_ex_noalloc(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Hk: int, M: int, N: int,
                       D: int, scale: float, causal: int, dtype: int, n_splits: int, stream: int | None) -> int:
    """Direct call of the allocation-free C entry point (split partials in the
    library's static device scratch array); pointers are integers.  Returns
    the fa2_status code."""
    return int(_lib.fa2_fwd_ex_noalloc(q, k, v, o, lse, B, H, Hk, M, N, D, scale, causal, dtype, n_splits,
                                       stream))


def fa2_fwd_workspace_bytes(B: int, H: int, M: int, D: int, n_splits: int) -> int:
    return int(_lib.fa2_fwd_workspace_bytes(B, H, M, D, n_splits))


def fa2_fwd_num_splits(B: int, H: int, Hk: int, M: int, N: int, D: int, causal: int, dtype: int) -> int:
    return int(_lib.fa2_fwd_num_splits(B, H, Hk, M, N, D, causal, dtype))


def fa2_fwd_local(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Hk: int, M: int, N: int, D: int,
                  scale: float, causal: int, window_left: int, window_right: int, dtype: int,
                  stream: int | None) -> int:
    """Direct call of the sliding-window C entry point; pointers are integers.
    Returns the fa2_status code."""
    return int(_lib.fa2_fwd_local(q, k, v, o, lse, B, H, Hk, M, N, D, scale, causal, window_left,
                                  window_right, dtype, stream))


def fa2_fwd_varlen(q: int, k: int, v: int, o: int, lse: int, cu_seqlens_q: int, cu_seqlens_k: int, B: int,
                   H: int, Hk: int, total_q: int, total_k: int, max_seqlen_q: int, D: int, scale: float,
                   causal: int, window_left: int, window_right: int, dtype: int, stream: int | None) -> int:
    """Direct call of the packed-sequence C entry point; pointers are
    integers.  Returns the fa2_status code."""
    return int(_lib.fa2_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, Hk, total_q, total_k,
                                   max_seqlen_q, D, scale, causal, window_left, window_right, dtype, stream))


def fa2_bwd(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int, delta: int,
            B: int, H: int, Hk: int, M: int, N: int, D: int, scale: float, causal: int, dtype: int,
            stream: int | None) -> int:
    """Direct call of the backward C entry point; pointers are integers.
    Returns the fa2_status code."""
    return int(_lib.fa2_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hk, M, N, D, scale, causal,
                            dtype, stream))


def fa2_bwd_local(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int, delta: int,
                  B: int, H: int, Hk: int, M: int, N: int, D: int, scale: float, causal: int, window_left: int,
                  window_right: int, dtype: int, stream: int | None) -> int:
    """Direct call of the sliding-window backward C entry point."""
    return int(_lib.fa2_bwd_local(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hk, M, N, D, scale, causal,
                                  window_left, window_right, dtype, stream))


def fa2_bwd_varlen(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int, delta: int,
                   cu_seqlens_q: int, cu_seqlens_k: int, B: int, H: int, Hk: int, total_q: int, total_k: int,
                   max_seqlen_q: int, max_seqlen_k: int, D: int, scale: float, causal: int, window_left: int,
                   window_right: int, dtype: int, stream: int | None) -> int:
    """Direct call of the packed-sequence backward C entry point."""
    return int(_lib.fa2_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, delta, cu_seqlens_q, cu_seqlens_k, B, H,
                                   Hk, total_q, total_k, max_seqlen_q, max_seqlen_k, D, scale, causal,
                                   window_left, window_right, dtype, stream))


def fa2_status_string(status: int) -> str:
    return _lib.fa2_status_string(int(status)).decode()


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return FA2_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return FA2_DTYPE_BF16
    if t.dtype == torch.float16:
        return FA2_DTYPE_F16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32, bfloat16 or float16")


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
            n_splits: int = 1, workspace=None, window=(-1, -1)):
    """Attention forward on the current CUDA/HIP stream.

    q: [B,H,M,D], k/v: [B,Hk,N,D] contiguous device tensors of one dtype
    (float32, bfloat16 or float16), H % Hk == 0 (query head h reads K/V head
    h // (H // Hk)).  Returns (o [B,H,M,D] in q's dtype, lse [B,H,M]
    float32).  ``scale`` defaults to 1/sqrt(D).  ``n_splits``: 1 = one kernel
    over all keys, 0 = library's choice, >1 = split K/V with a combine kernel;
    the workspace it needs is allocated with torch unless ``workspace`` (a
    device tensor of at least ``fa2_fwd_workspace_bytes`` bytes) is given.
    ``window`` = (left, right): sliding window (fa2_fwd_local; -1 leaves a
    side unbounded); it cannot be combined with split K/V.
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D tensor")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, H, M, D = q.shape
    Hk, N = k.shape[1], k.shape[2]
    if k.shape != (B, Hk, N, D) or v.shape != (B, Hk, N, D) or Hk < 1 or H % Hk:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer(out, q.shape, q.dtype, q.device, "out")
    if lse is None:
        lse = torch.empty((B, H, M), dtype=torch.float32, device=q.device)
    else:
        _check_buffer(lse, (B, H, M), torch.float32, q.device, "lse")
    code = _dtype_code(q)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    wl, wr = int(window[0]), int(window[1])
    if (wl, wr) != (-1, -1):
        if n_splits != 1:
            raise ValueError("a sliding window runs unsplit (n_splits=1)")
        with torch.cuda.device(q.device):
            st = fa2_fwd_local(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               B, H, Hk, M, N, D, float(scale), int(bool(causal)), wl, wr, code, stream)
        if st != FA2_OK:
            raise Fa2Error(st)
        return out, lse
    splits = fa2_fwd_num_splits(B, H, Hk, M, N, D, int(bool(causal)), code) if n_splits == 0 else int(n_splits)
    ws_ptr, ws_size = None, 0
    if splits > 1:
        need = fa2_fwd_workspace_bytes(B, H, M, D, splits)
        if need < 0:
            raise ValueError(f"invalid split count {splits}")
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        ws_ptr, ws_size = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = fa2_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        B, H, Hk, M, N, D, float(scale), int(bool(causal)), code, splits,
                        ws_ptr, ws_size, stream)
    if st != FA2_OK:
        raise Fa2Error(st)
    return out, lse


def _check_buffer(t, shape, dtype, device, name):
    """A caller-supplied output: the C entry points size their writes from the
    problem's shape, so a buffer that is short, of another type, strided or on
    another device is refused before any launch."""
    import torch
    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype
            or not t.is_contiguous() or t.device != device):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {list(shape)} on {device}")


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal: bool = False,
                   scale: float | None = None, window=(-1, -1), out=None, lse=None):
    """Forward over packed variable-length sequences (fa2_fwd_varlen).

    q: [H, total_q, D], k/v: [Hk, total_k, D] contiguous device tensors of one
    dtype; cu_seqlens_q / cu_seqlens_k: int32 device tensors of B + 1
    offsets (sequence b owns rows cu[b] .. cu[b+1]-1 of every head);
    max_seqlen_q bounds every sequence's query count.  Returns
    (o [H, total_q, D], lse [H, total_q] float32).
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 3-D tensor [heads, total, D]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if (not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int32 or t.dim() != 1
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous 1-D int32 device tensor")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must hold the same number (B + 1) of offsets")
    H, total_q, D = q.shape
    Hk, total_k = k.shape[0], k.shape[1]
    if k.shape != (Hk, total_k, D) or v.shape != k.shape or Hk < 1 or H % Hk:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    B = cu_seqlens_q.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer(out, q.shape, q.dtype, q.device, "out")
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    else:
        _check_buffer(lse, (H, total_q), torch.float32, q.device, "lse")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = fa2_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, Hk, total_q, total_k,
                            int(max_seqlen_q), D, float(scale), int(bool(causal)), int(window[0]),
                            int(window[1]), _dtype_code(q), stream)
    if st != FA2_OK:
        raise Fa2Error(st)
    return out, lse


def backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
             dq=None, dk=None, dv=None, delta=None, window=(-1, -1)):
    """Gradients of the attention forward on the current CUDA/HIP stream.

    q, o, dout: [B,H,M,D]; k, v: [B,Hk,N,D], contiguous device tensors of one
    dtype (float32, bfloat16 or float16); lse: the forward's [B,H,M] float32 output
    for the same inputs, scale and causal flag.  Returns (dq, dk, dv), shaped
    and typed like q, k, v; dk and dv sum over the query heads of each K/V
    head.  ``delta`` ([B,H,M] float32, rowsum(dout * o)) is scratch the call
    writes; it is allocated with torch unless given.  ``window``: the
    sliding window the forward used (fa2_bwd_local).
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D tensor")
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, o and dout must share one dtype")
    B, H, M, D = q.shape
    Hk, N = k.shape[1], k.shape[2]
    if (k.shape != (B, Hk, N, D) or v.shape != (B, Hk, N, D) or o.shape != q.shape
            or dout.shape != q.shape or Hk < 1 or H % Hk):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)} "
                         f"o{tuple(o.shape)} dout{tuple(dout.shape)}")
    if (not isinstance(lse, torch.Tensor) or lse.shape != (B, H, M) or lse.dtype != torch.float32
            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor of shape [B,H,M]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)

    def _out(t, like, name):
        if t is None:
            return torch.empty_like(like)
        _check_buffer(t, like.shape, like.dtype, like.device, name)
        return t

    dq, dk, dv = _out(dq, q, "dq"), _out(dk, k, "dk"), _out(dv, v, "dv")
    if delta is None:
        delta = torch.empty((B, H, M), dtype=torch.float32, device=q.device)
    else:
        _check_buffer(delta, (B, H, M), torch.float32, q.device, "delta")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = fa2_bwd_local(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                           B, H, Hk, M, N, D, float(scale), int(bool(causal)), int(window[0]), int(window[1]),
                           _dtype_code(q), stream)
    if st != FA2_OK:
        raise Fa2Error(st)
    return dq, dk, dv


def backward_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    causal: bool = False, scale: float | None = None, window=(-1, -1)):
    """Gradients of forward_varlen: q, o, dout [H, total_q, D]; k, v
    [Hk, total_k, D]; lse [H, total_q] from forward_varlen with the same
    offsets, causal flag, window and scale.  Returns (dq, dk, dv)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 3-D device tensor [heads, total, D]")
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, o and dout must share one dtype")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if (not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int32 or t.dim() != 1
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous 1-D int32 device tensor")
    H, total_q, D = q.shape
    Hk, total_k = k.shape[0], k.shape[1]
    if (k.shape != (Hk, total_k, D) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape
            or Hk < 1 or H % Hk or cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1):
        raise ValueError("shape mismatch between q, k, v, o, dout and the offsets")
    if lse.shape != (H, total_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape [H, total_q]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = fa2_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                            cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), cu_seqlens_q.numel() - 1, H, Hk,
                            total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), D, float(scale),
                            int(bool(causal)), int(window[0]), int(window[1]), _dtype_code(q), stream)
    if st != FA2_OK:
        raise Fa2Error(st)
    return dq, dk, dv


def _make_function():
    import torch

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, scale, window):
            o, lse = forward(q, k, v, causal=causal, scale=scale, window=window)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.causal, ctx.scale, ctx.window = causal, scale, window
            return o

        @staticmethod
        def backward(ctx, dout):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv = backward(q, k, v, o, lse, dout.contiguous(), causal=ctx.causal, scale=ctx.scale,
                                  window=ctx.window)
            return dq, dk, dv, None, None, None

    return _Attention


_function = None


def attention(q, k, v, causal: bool = False, scale: float | None = None, window=(-1, -1)):
    """softmax(scale * q k^T) v with autograd: the forward runs fa2_fwd_ex
    (fa2_fwd_local with a window), the backward fa2_bwd_local."""
    global _function
    if _function is None:
        _function = _make_function()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _function.apply(q, k, v, bool(causal), float(scale), (int(window[0]), int(window[1])))
