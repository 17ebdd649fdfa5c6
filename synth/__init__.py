"""Seeded synthetic inputs for the gated-delta-rule forward pass.

This module is shared by the HIP path's tests/benchmark and by the oracle's
tests.  It holds none of the recurrence's arithmetic: only random draws, the
input transforms that define the workloads (per-head-vector L2 normalisation
of q and k, sigmoid for beta, negative softplus for the log-decay g) and the
storage casts (float32 round-to-nearest-even, then bfloat16
round-to-nearest-even).

Workloads follow the HyMo pages' GDN interface: q/k are (B,T,H,dk), v is
(B,T,H,dv), g and beta are (B,T,H) ("Optimization Quartet", section 3.2, the
recurrence in math), with chunk length 64 by default ("v1.0 Architecture &
Design Spec", section 2.3).  The pages test their kernel on random inputs
("v1.0 Architecture & Design Spec", section 12a.1), so seeded synthetic
tensors are the workload itself.

Recipe (every draw is float64 from ``numpy.random.default_rng(seed)``, in
this order): varlen lengths (packed workload only) -> q -> k -> v ->
beta pre-activation -> g pre-activation -> h0 (only when the workload has a
non-zero initial state).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, dtype and distribution description of one synthetic workload."""

    name: str
    seed: int
    B: int                      # batch (dense) or number of sequences (varlen)
    T: int                      # tokens per sequence (dense) or packed total (varlen)
    H: int
    dk: int
    dv: int
    dtype: str                  # storage dtype of q/k/v/out: "f32" or "bf16"
    chunk: int
    h0_std: float = 0.0         # 0 -> no initial state (h0 = NULL)
    g_mean: float = 0.0         # g = -softplus(N(g_mean, 1))
    no_decay: bool = False      # g = 0 (its draw is still taken, so the other draws are unchanged)
    varlen: bool = False
    len_lo: int = 0             # varlen: lengths ~ U[len_lo, len_hi] (inclusive)
    len_hi: int = 0
    nseq: int = 0
    seq_lens: tuple = ()        # varlen with fixed lengths (no length draw)

    @property
    def tokens(self) -> int:
        return self.T if self.varlen else self.B * self.T


def _varlen(name, seed, nseq, lo, hi, H, dk, dv, dtype, chunk, **kw):
    lens = np.random.default_rng(seed).integers(lo, hi + 1, size=nseq)
    return Workload(name=name, seed=seed, B=nseq, T=int(lens.sum()), H=H, dk=dk,
                    dv=dv, dtype=dtype, chunk=chunk, varlen=True, len_lo=lo,
                    len_hi=hi, nseq=nseq, **kw)


#: The workloads, indexed by seed.
WORKLOADS = {
    "tiny": Workload("tiny", 0, B=1, T=64, H=2, dk=32, dv=32, dtype=F32, chunk=16),
    "small_state": Workload("small_state", 1, B=8, T=4096, H=16, dk=32, dv=32,
                            dtype=BF16, chunk=64),
    "wide_head": Workload("wide_head", 2, B=4, T=4096, H=16, dk=128, dv=128,
                          dtype=BF16, chunk=64, h0_std=0.02),
    "varlen": _varlen("varlen", 3, 32, 256, 4096, H=16, dk=128, dv=128,
                      dtype=BF16, chunk=64),
    "long_context": Workload("long_context", 4, B=1, T=32768, H=16, dk=128,
                             dv=128, dtype=BF16, chunk=64, g_mean=-2.0),
    # long_context without any decay: a segment's halo would reach back to
    # the sequence start, the case the chunk-map scan is for.
    "long_context_nodecay": Workload("long_context_nodecay", 6, B=1, T=32768, H=16, dk=128,
                                     dv=128, dtype=BF16, chunk=64, no_decay=True),
    # One decoding step at batch scale (the token-by-token entry point's
    # workload): the traffic is dominated by the state read and write.
    "decode": Workload("decode", 5, B=128, T=1, H=16, dk=128, dv=128, dtype=BF16,
                       chunk=64, h0_std=0.02),
}


def custom(name="custom", seed=0, B=1, T=64, H=2, dk=32, dv=32, dtype=F32,
           chunk=64, h0_std=0.0, g_mean=0.0, seq_lens=None, no_decay=False) -> Workload:
    """A workload with the standard distributions at arbitrary sizes.

    ``seq_lens`` (a sequence of ints) makes it a packed varlen workload with
    exactly those lengths; B and T are then derived from it.
    """
    if seq_lens is not None:
        lens = [int(x) for x in seq_lens]
        return Workload(name, seed, B=len(lens), T=sum(lens), H=H, dk=dk, dv=dv,
                        dtype=dtype, chunk=chunk, h0_std=h0_std, g_mean=g_mean,
                        no_decay=no_decay, varlen=True, nseq=len(lens), seq_lens=tuple(lens))
    return Workload(name, seed, B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype,
                    chunk=chunk, h0_std=h0_std, g_mean=g_mean, no_decay=no_decay)


# ---------------------------------------------------------------- casts ---

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern (uint16), round to nearest even.

    Inputs here are finite, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern (uint16) -> exact float64 values."""
    u = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


# ---------------------------------------------------------------- draws ---

def _l2norm(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


@dataclasses.dataclass
class Inputs:
    """Stored inputs of one workload.

    q, k, v are float32 arrays (``dtype == "f32"``) or uint16 bfloat16 bit
    patterns (``dtype == "bf16"``).  g, beta, h0 are float32.  Dense layout:
    q/k (B,T,H,dk), v (B,T,H,dv), g/beta (B,T,H).  Varlen layout: the same
    without the leading B (packed tokens), plus int32 ``cu_seqlens`` (B+1).
    h0 is (B,H,dk,dv) or None.
    """

    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    h0: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]

    def as_f64(self, name: str) -> np.ndarray:
        """Exact float64 view of a stored input (what the oracle consumes)."""
        x = getattr(self, name)
        if x is None:
            return None
        if x.dtype == np.uint16:
            return bf16_bits_to_f64(x)
        return x.astype(np.float64)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return f32_to_bf16_bits(x32) if dtype == BF16 else x32


def generate(wl: Workload) -> Inputs:
    """Draw the inputs of ``wl`` from ``default_rng(wl.seed)``.

    A varlen workload without fixed ``seq_lens`` first draws its lengths
    uniformly from [len_lo, len_hi] with the same generator.
    """
    rng = np.random.default_rng(wl.seed)
    cu = None
    if wl.varlen:
        if wl.seq_lens:
            lens = np.asarray(wl.seq_lens, dtype=np.int64)
        else:
            lens = rng.integers(wl.len_lo, wl.len_hi + 1, size=wl.nseq)
        cu = np.zeros(len(lens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens)
        lead = (int(cu[-1]),)
    else:
        lead = (wl.B, wl.T)
    H, dk, dv = wl.H, wl.dk, wl.dv
    q = _l2norm(rng.standard_normal(lead + (H, dk)))
    k = _l2norm(rng.standard_normal(lead + (H, dk)))
    v = rng.standard_normal(lead + (H, dv))
    beta = _sigmoid(rng.standard_normal(lead + (H,)))
    g = -_softplus(rng.normal(wl.g_mean, 1.0, size=lead + (H,)))
    if wl.no_decay:
        g = np.zeros_like(g)
    h0 = None
    if wl.h0_std > 0:
        h0 = (rng.standard_normal((wl.B, H, dk, dv)) * wl.h0_std).astype(np.float32)
    return Inputs(wl=wl, q=_store(q, wl.dtype), k=_store(k, wl.dtype),
                  v=_store(v, wl.dtype), g=g.astype(np.float32),
                  beta=beta.astype(np.float32), h0=h0, cu_seqlens=cu)


def chain_bounds(inp: Inputs, n: int):
    """(token start, token end) of sequence ``n`` in the packed layout."""
    return int(inp.cu_seqlens[n]), int(inp.cu_seqlens[n + 1])


@dataclasses.dataclass
class OutputGrads:
    """Seeded gradients of the forward's outputs, for the backward pass.

    dout has out's layout and storage dtype (float32, or uint16 bfloat16 bit
    patterns); dhT is float32 (B, H, dk, dv) or None.
    """

    dout: np.ndarray
    dhT: Optional[np.ndarray]

    def as_f64(self, name: str) -> Optional[np.ndarray]:
        x = getattr(self, name)
        if x is None:
            return None
        if x.dtype == np.uint16:
            return bf16_bits_to_f64(x)
        return x.astype(np.float64)


def output_grads(inp: Inputs, seed: int, dhT_std: float = 1.0) -> OutputGrads:
    """dout ~ N(0, 1) in v's shape and dtype, dhT ~ N(0, dhT_std^2) (None
    when ``dhT_std`` is 0), drawn from ``default_rng(seed)`` in that order."""
    rng = np.random.default_rng(seed)
    wl = inp.wl
    dout = _store(rng.standard_normal(inp.v.shape), wl.dtype)
    dhT = None
    if dhT_std > 0:
        dhT = (rng.standard_normal((wl.B, wl.H, wl.dk, wl.dv)) * dhT_std).astype(np.float32)
    return OutputGrads(dout=dout, dhT=dhT)
