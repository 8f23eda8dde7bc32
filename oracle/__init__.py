"""CPU oracle for the attention forward and backward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never links,
loads or calls it, and it shares no code with the HIP path.

The arithmetic lives in ``fa2_oracle.c`` (plain C, IEEE double, one score
row at a time, no -ffast-math).  This module only builds that file with gcc
and marshals arrays into it through ctypes.

Every function of the oracle is pinned by ``tests/test_oracle.py`` to closed
forms, invariants, a library special case and a 50-digit brute force (the
backward also to central finite differences of the forward); none is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa2_oracle.c")
_LIB = os.path.join(_HERE, "libfa2_oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile fa2_oracle.c into oracle/libfa2_oracle.so with gcc."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", _LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _bind(lib):
    lib.fa2_oracle_fwd.restype = ctypes.c_int
    lib.fa2_oracle_fwd.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
    ]
    lib.fa2_oracle_fwd_gqa.restype = ctypes.c_int
    lib.fa2_oracle_fwd_gqa.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
    ]
    lib.fa2_oracle_fwd_local.restype = ctypes.c_int
    lib.fa2_oracle_fwd_local.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_int,
    ]
    lib.fa2_oracle_bwd_gqa.restype = ctypes.c_int
    lib.fa2_oracle_bwd_gqa.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_double, ctypes.c_int, ctypes.c_int,
    ]
    lib.fa2_oracle_bwd_local.restype = ctypes.c_int
    lib.fa2_oracle_bwd_local.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
    ]
    lib.fa2_oracle_max_threads.restype = ctypes.c_int
    lib.fa2_oracle_max_threads.argtypes = []
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def max_threads() -> int:
    return int(_load().fa2_oracle_max_threads())


def _as_f32(x) -> np.ndarray:
    """Exact float32 carrier of the input values (fp32 as is, bf16/fp16 widened)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu")
            if x.dtype not in (torch.float32, torch.bfloat16, torch.float16):
                raise TypeError(f"oracle inputs must be float32, bfloat16 or float16, got {x.dtype}")
            x = x.to(torch.float32).contiguous().numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    a = np.asarray(x)
    if a.dtype != np.float32:
        raise TypeError(f"oracle inputs must carry float32 values, got {a.dtype}")
    return np.ascontiguousarray(a)


def attention(q, k, v, scale: float, causal: bool, rows: Optional[np.ndarray] = None,
              threads: int = 0, _lib_override=None, window=(-1, -1)):
    """Reference attention forward.

    q: [B,H,M,D], k/v: [B,Hk,N,D] with H % Hk == 0 (torch tensors or float32
    numpy arrays); query head h reads K/V head h // (H // Hk).
    rows: optional int64 array of query rows (same for every head); when
    given, outputs cover only those rows.
    window: (left, right) sliding window; query row i sees keys
    i - left <= j <= i + right (a negative side is unbounded), on top of
    the causal mask.  Rows that see no key get O = 0 and L = -inf.
    Returns (o, lse) as float64 numpy arrays: o [B,H,R,D], lse [B,H,R].
    """
    qa, ka, va = _as_f32(q), _as_f32(k), _as_f32(v)
    if qa.ndim != 4 or ka.ndim != 4 or va.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B,H,seq,D]")
    B, H, M, D = qa.shape
    Hk, N = ka.shape[1], ka.shape[2]
    if ka.shape != (B, Hk, N, D) or va.shape != (B, Hk, N, D) or Hk < 1 or H % Hk:
        raise ValueError(f"shape mismatch q{qa.shape} k{ka.shape} v{va.shape}")
    if rows is not None:
        rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        R = rows_a.shape[0]
        rows_p = rows_a.ctypes.data
    else:
        rows_a = None
        R = M
        rows_p = None
    o = np.empty((B, H, R, D), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    lib = _load() if _lib_override is None else _lib_override
    wl, wr = (int(window[0]), int(window[1]))
    if wl >= 0 or wr >= 0:
        rc = lib.fa2_oracle_fwd_local(qa.ctypes.data, ka.ctypes.data, va.ctypes.data,
                                      o.ctypes.data, lse.ctypes.data, B, H, Hk, M, N, D,
                                      float(scale), int(bool(causal)), wl, wr, rows_p, R, int(threads))
    elif Hk == H:
        rc = lib.fa2_oracle_fwd(qa.ctypes.data, ka.ctypes.data, va.ctypes.data,
                                o.ctypes.data, lse.ctypes.data, B, H, M, N, D,
                                float(scale), int(bool(causal)), rows_p, R, int(threads))
    else:
        rc = lib.fa2_oracle_fwd_gqa(qa.ctypes.data, ka.ctypes.data, va.ctypes.data,
                                    o.ctypes.data, lse.ctypes.data, B, H, Hk, M, N, D,
                                    float(scale), int(bool(causal)), rows_p, R, int(threads))
    if rc != 0:
        raise ValueError(f"fa2_oracle_fwd failed with status {rc}")
    del rows_a
    return o, lse


def attention_bwd_varlen(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool,
                         window=(-1, -1), threads: int = 0):
    """Reference gradients over packed sequences (layout of
    ``attention_varlen``): each sequence's rows through ``attention_bwd``
    (no arithmetic here).  Returns (dq [H,total_q,D], dk, dv [Hk,total_k,D])
    in float64; keys of no sequence keep a zero gradient."""
    qa, ka, va, da = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(dout)
    cq = [int(x) for x in np.asarray(cu_seqlens_q).tolist()]
    ck = [int(x) for x in np.asarray(cu_seqlens_k).tolist()]
    dq = np.zeros(qa.shape, dtype=np.float64)
    dk = np.zeros(ka.shape, dtype=np.float64)
    dv = np.zeros(va.shape, dtype=np.float64)
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 <= q0 or k1 <= k0:
            continue
        g = attention_bwd(qa[None, :, q0:q1], ka[None, :, k0:k1], va[None, :, k0:k1], da[None, :, q0:q1],
                          scale, causal, threads=threads, window=window)
        dq[:, q0:q1], dk[:, k0:k1], dv[:, k0:k1] = g[0][0], g[1][0], g[2][0]
    return dq, dk, dv


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool,
                     window=(-1, -1), threads: int = 0):
    """Reference forward over packed variable-length sequences.

    q: [H, total_q, D], k/v: [Hk, total_k, D]; sequence b owns query rows
    cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 and keys cu_seqlens_k[b] ..
    cu_seqlens_k[b+1] - 1 of every head, and attends only within itself.
    Each sequence is evaluated by ``attention`` on its own rows (no
    arithmetic here).  Returns (o [H,total_q,D], lse [H,total_q]) in
    float64.
    """
    qa, ka, va = _as_f32(q), _as_f32(k), _as_f32(v)
    cq = [int(x) for x in np.asarray(cu_seqlens_q).tolist()]
    ck = [int(x) for x in np.asarray(cu_seqlens_k).tolist()]
    if qa.ndim != 3 or ka.ndim != 3 or va.ndim != 3 or len(cq) != len(ck) or len(cq) < 1:
        raise ValueError("q, k, v must be [heads, total, D] with matching cu_seqlens")
    H, total_q, D = qa.shape
    o = np.zeros((H, total_q, D), dtype=np.float64)
    lse = np.full((H, total_q), -np.inf, dtype=np.float64)
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 <= q0:
            continue
        if k1 <= k0:  # no keys: every row sees nothing
            continue
        ob, lb = attention(qa[None, :, q0:q1], ka[None, :, k0:k1], va[None, :, k0:k1], scale, causal,
                           threads=threads, window=window)
        o[:, q0:q1] = ob[0]
        lse[:, q0:q1] = lb[0]
    return o, lse


def attention_bwd(q, k, v, dout, scale: float, causal: bool, threads: int = 0, _lib_override=None,
                  window=(-1, -1)):
    """Reference gradients of the attention forward for the upstream gradient
    dout: q, dout [B,H,M,D]; k, v [B,Hk,N,D].  Returns (dq, dk, dv) as float64
    numpy arrays shaped like q, k, v; dk and dv sum over the query heads of
    each K/V head.  ``window``: the forward's sliding window (see
    ``attention``); rows that see no key have no gradient."""
    qa, ka, va, da = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(dout)
    B, H, M, D = qa.shape
    Hk, N = ka.shape[1], ka.shape[2]
    if (ka.shape != (B, Hk, N, D) or va.shape != (B, Hk, N, D) or da.shape != qa.shape
            or Hk < 1 or H % Hk):
        raise ValueError(f"shape mismatch q{qa.shape} k{ka.shape} v{va.shape} dout{da.shape}")
    dq = np.empty((B, H, M, D), dtype=np.float64)
    dk = np.empty((B, Hk, N, D), dtype=np.float64)
    dv = np.empty((B, Hk, N, D), dtype=np.float64)
    lib = _load() if _lib_override is None else _lib_override
    wl, wr = int(window[0]), int(window[1])
    if wl >= 0 or wr >= 0:
        rc = lib.fa2_oracle_bwd_local(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, da.ctypes.data,
                                      dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
                                      B, H, Hk, M, N, D, float(scale), int(bool(causal)), wl, wr, int(threads))
    else:
        rc = lib.fa2_oracle_bwd_gqa(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, da.ctypes.data,
                                    dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
                                    B, H, Hk, M, N, D, float(scale), int(bool(causal)), int(threads))
    if rc != 0:
        raise ValueError(f"fa2_oracle_bwd_gqa failed with status {rc}")
    return dq, dk, dv
