"""Seeded synthetic attention workloads.

This module only draws random inputs and names the shapes; it holds none of
the attention arithmetic.  Both the HIP path's tests/bench and the CPU oracle
take their inputs from here, so the two sides always see identical values.

Recipe (the pages measure on seeded ``torch.randn`` tensors only, never on a
dataset -- "FlashAttention-2 from PyTorch to Triton", test and bench harness
listings; "Writing FlashAttention 2 in Triton", numerics verification
harness):

* a CPU ``torch.Generator`` seeded with ``seed`` draws Q, then K, then V as
  float32 standard normals of the full [B,H,M,D] / [B,H,N,D] shapes;
* Q and K are multiplied by ``qk_sigma`` and V by ``v_sigma`` (both 1 unless
  a workload stresses the max subtraction);
* for bf16 workloads the float32 draws are rounded to bfloat16 with
  round-to-nearest-even (``Tensor.to``).  The oracle then consumes exactly
  those rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

__all__ = ["Workload", "WORKLOADS", "ORDER", "WIDENED", "BACKWARD", "get", "make_inputs", "make_dout", "torch_dtype",
           "visible_pairs", "workload_inputs", "cu_seqlens"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    M: int
    N: int
    D: int
    dtype: str          # "f32", "bf16" or "f16"
    causal: bool
    qk_sigma: float = 1.0
    v_sigma: float = 1.0
    seed: int = 0
    # number of query rows per head checked against the oracle; None = all
    sample_rows: Optional[int] = None
    # K/V heads (grouped-query attention); None = H
    Hk: Optional[int] = None
    # K/V splits the bench asks for (0 = the library's choice, 1 = unsplit)
    n_splits: int = 1
    # sliding window (left, right); -1 leaves a side unbounded
    window: tuple = (-1, -1)
    # packed variable-length batch: per-sequence lengths (queries = keys);
    # None = the dense [B, H, M, D] layout.  With lengths, B is their count and
    # M, N are the longest one.
    lengths: Optional[tuple] = None

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hk is None else self.Hk

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> float:
        """Counted work 4*B*H*M*N*D, halved when causal.

        This is the accounting of the bench harness in "FlashAttention-2 from
        PyTorch to Triton" (two matmuls of M*N*D multiply-adds, halved for
        causal), generalised to M != N.  With a sliding window or packed
        sequences the M*N (or M*N/2) term becomes the number of visible
        (query, key) pairs.
        """
        if self.window == (-1, -1) and self.lengths is None:
            f = 4.0 * self.B * self.H * self.M * self.N * self.D
            return f / 2 if self.causal else f
        lens = self.lengths if self.lengths is not None else (self.M,) * self.B
        kl = self.lengths if self.lengths is not None else (self.N,) * self.B
        pairs = sum(visible_pairs(m, n, self.causal, *self.window) for m, n in zip(lens, kl))
        return 4.0 * self.H * self.D * pairs

    @property
    def bwd_flops(self) -> float:
        """Counted work of the backward pass: its five products (S recomputed,
        dP, dV, dK, dQ) of 2*M*N*D flop each per head, i.e. 2.5 times the
        forward's count, halved when causal."""
        return 2.5 * self.flops

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def compulsory_bytes(self) -> int:
        """Read Q, K, V once and write O and the fp32 logsumexp once."""
        if self.lengths is not None:
            total = sum(self.lengths)
            return ((self.H * 2 + self.kv_heads * 2) * total * self.D) * self.elt_bytes + 4 * self.H * total
        bh = self.B * self.H
        kv = self.B * self.kv_heads * 2 * self.N * self.D
        return (bh * 2 * self.M * self.D + kv) * self.elt_bytes + 4 * bh * self.M

    def describe(self) -> str:
        hk = "" if self.Hk is None else f",Hk={self.Hk}"
        return (f"{self.name}: B={self.B},H={self.H}{hk},M={self.M},N={self.N},D={self.D},"
                f"{self.dtype},{'causal' if self.causal else 'non-causal'}")


def visible_pairs(M: int, N: int, causal: bool, wl: int = -1, wr: int = -1) -> int:
    """Number of (query, key) pairs a query row i < M and key j < N form
    when j must satisfy i - wl <= j <= i + wr (a side is unbounded when -1)
    and j <= i when causal -- the rows' visible key counts, summed."""
    import numpy as np
    i = np.arange(M, dtype=np.int64)
    lo = np.zeros(M, dtype=np.int64) if wl < 0 else np.maximum(0, i - wl)
    hi = np.full(M, N - 1, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, i)
    if wr >= 0:
        hi = np.minimum(hi, i + wr)
    return int(np.maximum(hi - lo + 1, 0).sum())


def _varlen_lengths(count: int, lo: int, hi: int, seed: int) -> tuple:
    """Seeded sequence lengths, uniform in [lo, hi]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (count,), generator=g))


WORKLOADS = {
    # tiny fp32 self-attention, the case the oracle runs in full in milliseconds
    "tiny_f32": Workload("tiny_f32", 1, 1, 128, 128, 64, "f32", False, seed=1),
    # the fp32 shape the CUDA project page benchmarks (B=4,H=12,M=N=2048,D=64)
    "mha_f32_2k": Workload("mha_f32_2k", 4, 12, 2048, 2048, 64, "f32", False, seed=2),
    # causal bf16, head dim 128
    "causal_bf16_4k": Workload("causal_bf16_4k", 4, 16, 4096, 4096, 128, "bf16", True, seed=3),
    # long-context causal bf16; the oracle checks a seeded sample of 512 rows per head
    "causal_bf16_16k": Workload("causal_bf16_16k", 1, 32, 16384, 16384, 128, "bf16", True,
                                seed=4, sample_rows=512),
    # ragged cross-attention; Q,K ~ N(0, 4^2) so scores reach ~90 (past fp32 exp overflow)
    "ragged_bf16_cross": Workload("ragged_bf16_cross", 8, 8, 1000, 3000, 64, "bf16", False,
                                  qk_sigma=4.0, seed=5),
}

ORDER = ["tiny_f32", "mha_f32_2k", "causal_bf16_4k", "causal_bf16_16k", "ragged_bf16_cross"]

# The widened rows (grouped-query heads, fp16, split K/V), measured and
# checked like the workloads above but not part of the headline set.
WORKLOADS.update({
    # the causal 4k shape with fp16 inputs
    "causal_f16_4k": Workload("causal_f16_4k", 4, 16, 4096, 4096, 128, "f16", True, seed=6),
    # the causal 4k shape with 4 query heads per K/V head
    "gqa_bf16_4k": Workload("gqa_bf16_4k", 4, 16, 4096, 4096, 128, "bf16", True, seed=7, Hk=4),
    # decode-like: 16 new query rows per head against a 16k-key cache, 4 query
    # heads per K/V head, split K/V chosen by the library
    "decode_gqa_bf16": Workload("decode_gqa_bf16", 4, 32, 16, 16384, 128, "bf16", False, seed=8,
                                Hk=8, n_splits=0),
})
WORKLOADS.update({
    # the long-context causal shape with a 4096-key sliding window (each row
    # sees itself and the 4095 keys before it)
    "swa_bf16_16k": Workload("swa_bf16_16k", 1, 32, 16384, 16384, 128, "bf16", True, seed=9,
                             window=(4095, 0), sample_rows=512),
})
_VL = _varlen_lengths(16, 128, 8192, seed=10)
WORKLOADS.update({
    # 16 packed causal sequences of 128..8192 tokens (seeded lengths), 4
    # query heads per K/V head
    "varlen_bf16_mix": Workload("varlen_bf16_mix", len(_VL), 16, max(_VL), max(_VL), 128, "bf16", True,
                                seed=10, Hk=4, lengths=_VL),
})
WIDENED = ["causal_f16_4k", "gqa_bf16_4k", "decode_gqa_bf16", "swa_bf16_16k", "varlen_bf16_mix"]

# Workloads whose backward pass the bench also times.
BACKWARD = ["causal_bf16_4k", "causal_bf16_16k", "ragged_bf16_cross", "gqa_bf16_4k", "causal_f16_4k", "mha_f32_2k"]


def get(name: str) -> Workload:
    return WORKLOADS[name]


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def make_inputs(B: int, H: int, M: int, N: int, D: int, dtype: str = "f32", seed: int = 0,
                qk_sigma: float = 1.0, v_sigma: float = 1.0, Hk: int | None = None):
    """Draw (q, k, v) on the CPU, contiguous, in the I/O dtype (rounded to
    nearest even from fp32 draws).  k and v have Hk heads (default H)."""
    Hk = H if Hk is None else Hk
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, H, M, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hk, N, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hk, N, D), generator=g, dtype=torch.float32)
    if qk_sigma != 1.0:
        q.mul_(qk_sigma)
        k.mul_(qk_sigma)
    if v_sigma != 1.0:
        v.mul_(v_sigma)
    td = torch_dtype(dtype)
    if td != torch.float32:
        q, k, v = q.to(td), k.to(td), v.to(td)
    return q.contiguous(), k.contiguous(), v.contiguous()


def workload_inputs(w: Workload):
    """(q, k, v) of a workload: dense [B,H,M,D] / [B,Hk,N,D], or for packed
    sequences [H, total, D] / [Hk, total, D] drawn as one long sequence."""
    if w.lengths is not None:
        total = sum(w.lengths)
        q, k, v = make_inputs(1, w.H, total, total, w.D, w.dtype, w.seed, w.qk_sigma, w.v_sigma, Hk=w.Hk)
        return q[0], k[0], v[0]
    return make_inputs(w.B, w.H, w.M, w.N, w.D, w.dtype, w.seed, w.qk_sigma, w.v_sigma, Hk=w.Hk)


def cu_seqlens(w: Workload):
    """int32 offsets [B + 1] of a packed workload's sequences."""
    import itertools
    return torch.tensor([0] + list(itertools.accumulate(w.lengths)), dtype=torch.int32)


def sample_rows(w: Workload, seed_offset: int = 1000):
    """Seeded per-workload sample of query rows (same rows for every head).

    Rows 0 and M-1 are always included; the rest are drawn uniformly without
    replacement.  Returns a sorted int64 tensor, or None when every row is
    checked.
    """
    if w.sample_rows is None or w.sample_rows >= w.M:
        return None
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + seed_offset)
    inner = torch.randperm(w.M - 2, generator=g)[: w.sample_rows - 2] + 1
    rows = torch.cat([torch.tensor([0, w.M - 1]), inner]).sort().values
    return rows.to(torch.int64)


def make_dout(B: int, H: int, M: int, D: int, dtype: str = "bf16", seed: int = 0, sigma: float = 1.0):
    """Seeded upstream gradient dO [B,H,M,D] for the backward pass: float32
    standard normals from their own CPU generator (seed + 7919, so dO never
    repeats the draws of Q), times ``sigma``, rounded to the I/O dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 7919)
    do = torch.randn((B, H, M, D), generator=g, dtype=torch.float32)
    if sigma != 1.0:
        do.mul_(sigma)
    td = torch_dtype(dtype)
    return (do.to(td) if td != torch.float32 else do).contiguous()
