"""Oracle for the affine chunk map of the gated delta rule (FP64, CPU).

TEST INFRASTRUCTURE ONLY.  Only the tests may import this module; the
product library never does, and this module imports nothing from it.

Over one chunk the rule is affine in the entry state (M = S^T, dk x dv):
M_next = P_c M + Q_c.  Unrolling the chunk form of the forward (the chunk
algebra of ``oracle.fwd_chunked``; HyMo "Model Architecture Walkthrough",
sections 5.2.1-5.2.2 for the rule, "v1.0 Architecture & Design Spec",
section 2.3 for the chunking) gives

    P_c = Gam_C I - (diag(w) K)^T W,    Q_c = (diag(w) K)^T Uh,
    W = (I + A)^-1 diag(beta Gam) K,    Uh = (I + A)^-1 diag(beta) V,

with A, Gam, w as there.  Maps compose: (P2, Q2) after (P1, Q1) is
(P2 P1, P2 Q1 + Q2).  A sequence cut into segments therefore gets every
segment's exact entry state from the segments' composed maps by a short
sequential scan -- the intra-sequence parallel form of the recurrence (and
of its sharding over GPUs).  Plain FP64 with ``numpy.linalg.inv``.
"""
from __future__ import annotations

import numpy as np


def chunk_map(k, v, g, beta):
    """(P, Q) of one chunk: k (C, dk), v (C, dv), g and beta (C,)."""
    k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (k, v, g, beta))
    C, dk = k.shape
    gam = np.cumsum(g)
    Gam = np.exp(gam)
    E = np.exp(gam[:, None] - gam[None, :])
    A = beta[:, None] * (k @ k.T) * E * np.tril(np.ones((C, C)), -1)
    Ti = np.linalg.inv(np.eye(C) + A)
    W = Ti @ ((beta * Gam)[:, None] * k)
    Uh = Ti @ (beta[:, None] * v)
    Kt = np.exp(gam[-1] - gam)[:, None] * k
    return Gam[-1] * np.eye(dk) - Kt.T @ W, Kt.T @ Uh


def compose(first, second):
    """The map of ``first`` followed by ``second``."""
    P1, Q1 = first
    P2, Q2 = second
    return P2 @ P1, P2 @ Q1 + Q2


def segment_maps(k, v, g, beta, chunk, seg_chunks):
    """Composed maps of consecutive segments of ``seg_chunks`` chunks of one
    chain (k (T, dk), v (T, dv), g and beta (T,)); the last may be shorter."""
    T = k.shape[0]
    maps = []
    for s0 in range(0, T, chunk * seg_chunks):
        acc = None
        for c0 in range(s0, min(s0 + chunk * seg_chunks, T), chunk):
            sl = slice(c0, min(c0 + chunk, T))
            m = chunk_map(k[sl], v[sl], g[sl], beta[sl])
            acc = m if acc is None else compose(acc, m)
        maps.append(acc)
    return maps


def scan_entry_states(maps, h0):
    """Entry state of every segment (and the final state) from h0 by the
    sequential scan M_{s+1} = P_s M_s + Q_s."""
    M = np.asarray(h0, dtype=np.float64)
    states = [M]
    for P, Q in maps:
        M = P @ M + Q
        states.append(M)
    return states
