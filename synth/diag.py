"""Seeded synthetic inputs for the diagonal-decay additive recurrence.

Shared by the HIP path's tests/benchmark and by the oracle's tests; holds
none of the recurrence's arithmetic, only random draws, the transforms that
define the input distributions and the storage casts of ``synth``.

Shapes follow the pages' kernel interface ("Optimization Quartet", section
3.2): v and out (B,T,H,D), write key b and read key c (B,T,H,S), the
per-head gate g (B,T,H), A_log (H,S); the block's epilogue adds D (H,) and
the output gate (B,T,H) ("Model Architecture Walkthrough", sections 5.5 and
5.6).  The HyMo layer runs it at B=4, T=4096, H=40, S=D=32 (section 5.5).

Recipe (float64 draws from ``numpy.random.default_rng(seed)``, in this
order; varlen lengths first when the workload is packed):

* v ~ N(0, 1)                         (values after the conv and SiLU)
* b, c ~ N(0, 1/S)                    (linear projections of those values)
* g = sigmoid(N(0, 1))                (positive per-head gate, Walkthrough 5.2.1)
* A_log[h, s] = log(h + 1) + N(0, 0.25^2)
      (the multi-scale initialisation of Walkthrough 5.3.2, one decay rate
      per head, with a per-key-row spread so that every row decays at its
      own rate)
* D[h] = 1 + N(0, 0.1^2)              (initialised to one, section 5.6)
* gate = sigmoid(N(0, 0.25^2))        (a per-head mean of sigmoids: near 0.5)
* h0 ~ N(0, h0_std^2) when h0_std > 0
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from synth import BF16, F32, _store


@dataclasses.dataclass(frozen=True)
class DiagWorkload:
    name: str
    seed: int
    B: int
    T: int
    H: int
    S: int
    D: int
    dtype: str
    h0_std: float = 0.0
    epilogue: bool = True        # draw D and gate
    seq_lens: tuple = ()         # packed workload with these lengths

    @property
    def varlen(self) -> bool:
        return bool(self.seq_lens)

    @property
    def tokens(self) -> int:
        return sum(self.seq_lens) if self.varlen else self.B * self.T


WORKLOADS = {
    "diag_tiny": DiagWorkload("diag_tiny", 20, B=2, T=37, H=3, S=32, D=32, dtype=F32,
                              h0_std=0.1),
    # The HyMo layer's shape (Walkthrough section 5.5): B=4, T=4096, 40 heads,
    # S = D = 32.
    "hymo": DiagWorkload("hymo", 21, B=4, T=4096, H=40, S=32, D=32, dtype=BF16),
    # One decoding step of the same layer at serving batch.
    "hymo_decode": DiagWorkload("hymo_decode", 22, B=256, T=1, H=40, S=32, D=32,
                                dtype=BF16, h0_std=0.1),
}


def custom(name="diag_custom", seed=0, B=1, T=64, H=2, S=32, D=32, dtype=F32,
           h0_std=0.0, epilogue=True, seq_lens=None) -> DiagWorkload:
    if seq_lens is not None:
        lens = tuple(int(x) for x in seq_lens)
        return DiagWorkload(name, seed, B=len(lens), T=sum(lens), H=H, S=S, D=D,
                            dtype=dtype, h0_std=h0_std, epilogue=epilogue,
                            seq_lens=lens)
    return DiagWorkload(name, seed, B=B, T=T, H=H, S=S, D=D, dtype=dtype,
                        h0_std=h0_std, epilogue=epilogue)


@dataclasses.dataclass
class DiagInputs:
    """Stored inputs: v, b, c float32 or bf16 bit patterns (uint16); g,
    A_log, Dskip, gate, h0 float32 (Dskip/gate/h0 may be None)."""

    wl: DiagWorkload
    v: np.ndarray
    b: np.ndarray
    c: np.ndarray
    g: np.ndarray
    A_log: np.ndarray
    Dskip: Optional[np.ndarray]
    gate: Optional[np.ndarray]
    h0: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]

    def as_f64(self, name: str):
        from synth import bf16_bits_to_f64

        x = getattr(self, name)
        if x is None:
            return None
        if x.dtype == np.uint16:
            return bf16_bits_to_f64(x)
        return x.astype(np.float64)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def generate(wl: DiagWorkload) -> DiagInputs:
    rng = np.random.default_rng(wl.seed)
    cu = None
    if wl.varlen:
        cu = np.zeros(len(wl.seq_lens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(wl.seq_lens)
        lead = (int(cu[-1]),)
    else:
        lead = (wl.B, wl.T)
    H, S, D = wl.H, wl.S, wl.D
    v = rng.standard_normal(lead + (H, D))
    b = rng.standard_normal(lead + (H, S)) / np.sqrt(S)
    c = rng.standard_normal(lead + (H, S)) / np.sqrt(S)
    g = _sigmoid(rng.standard_normal(lead + (H,)))
    A_log = np.log(np.arange(1, H + 1, dtype=np.float64))[:, None] + 0.25 * rng.standard_normal((H, S))
    Dskip = gate = None
    if wl.epilogue:
        Dskip = 1.0 + 0.1 * rng.standard_normal(H)
        gate = _sigmoid(0.25 * rng.standard_normal(lead + (H,)))
    h0 = None
    if wl.h0_std > 0:
        h0 = (rng.standard_normal((wl.B, H, S, D)) * wl.h0_std).astype(np.float32)
    f32 = lambda x: None if x is None else x.astype(np.float32)
    return DiagInputs(wl=wl, v=_store(v, wl.dtype), b=_store(b, wl.dtype), c=_store(c, wl.dtype),
                      g=f32(g), A_log=f32(A_log), Dskip=f32(Dskip), gate=f32(gate), h0=h0,
                      cu_seqlens=cu)
