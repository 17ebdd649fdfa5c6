"""Oracle for the diagonal-decay additive recurrence (FP64, CPU).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product library
never does, and this module imports nothing from it.

The recurrence HyMo writes for its GDN layer ("Model Architecture
Walkthrough", section 5.2.1; "Optimization Quartet", section 3.2), per
head, with a state H of shape (S, D) (S over the key dimension, D over the
value dimension):

    H_t = exp(g_t * A) (.) H_{t-1} + b_t (x) v_t        (decay per key row)
    o_t = c_t^T H_t                                       (read after write)

A = -exp(A_log) is the head's negative decay vector over S (section 5.2.1
gives A as strictly negative, minus the exponential of A_log; the
Quartet's A_log has shape (H, S)), g_t a positive per-head scalar.  The
epilogue the block applies right after the recurrence ("Model Architecture
Walkthrough", section 5.5 step 6 and section 5.6) is optional here:

    o_t <- (o_t + D_h v_t) * gate_t                       (D: (H,), gate: (B,T,H))

with either factor left out when it is not given.

Two independent evaluations, both float64:

* :func:`diag_fwd_seq` -- the token loop of section 5.5 step 5, vectorised
  over the independent chains (one state per sequence and head).
* :func:`diag_fwd_unrolled` -- the unrolled sum of section 5.3.1: the state
  at t is the initial state and every write b_tau (x) v_tau, each scaled by
  the product of the decays of the tokens after it, exp(A * sum g).  O(T^2)
  per chain, small inputs only.

Layouts (row-major): dense v, out (B,T,H,D); b, c (B,T,H,S); g, gate
(B,T,H); packed (``cu_seqlens`` given): the same without B.  A_log (H,S),
D (H,).  h0/hT (B,H,S,D) with hT[b,h,s,d] = H[s,d].
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _dims(v, b, cu_seqlens):
    if cu_seqlens is not None:
        T, H, D = v.shape
        B = len(cu_seqlens) - 1
    else:
        B, T, H, D = v.shape
    S = b.shape[-1]
    return B, T, H, S, D


def _chains(v, cu_seqlens):
    """Yield (sequence index, token index tuple) for every sequence."""
    if cu_seqlens is not None:
        for n in range(len(cu_seqlens) - 1):
            yield n, (slice(int(cu_seqlens[n]), int(cu_seqlens[n + 1])),)
    else:
        for n in range(v.shape[0]):
            yield n, (n,)


def epilogue(o, v, D=None, gate=None):
    """(o + D_h v) * gate_t, each factor applied only when given.

    Section 5.5 step 6 of the Walkthrough: the skip term D.view(1,1,H,1) * v,
    then the per-head gate broadcast over the value dimension.
    """
    o = np.array(o, dtype=np.float64)
    if D is not None:
        o = o + np.asarray(D, dtype=np.float64)[:, None] * np.asarray(v, dtype=np.float64)
    if gate is not None:
        o = o * np.asarray(gate, dtype=np.float64)[..., None]
    return o


def diag_fwd_seq(v, b, c, g, A_log, h0=None, cu_seqlens=None, D=None, gate=None):
    """Token loop of the recurrence.  Returns (out, hT) as float64 arrays.

    For each sequence the loop runs over its tokens with the states of all
    heads side by side: alpha = exp(g_t * A) (one factor per head and key
    row), H <- alpha H + b_t v_t^T, o_t = c_t^T H.
    """
    v, b, c, g, A_log, h0 = map(_f64, (v, b, c, g, A_log, h0))
    B, T, H, S, Dv = _dims(v, b, cu_seqlens)
    A = -np.exp(A_log)                                    # (H, S)
    out = np.zeros(v.shape, dtype=np.float64)
    hT = np.zeros((B, H, S, Dv), dtype=np.float64)
    for n, sel in _chains(v, cu_seqlens):
        st = np.zeros((H, S, Dv)) if h0 is None else h0[n].copy()
        V, Bk, Ck, G = v[sel], b[sel], c[sel], g[sel]     # (L,H,D) (L,H,S) (L,H,S) (L,H)
        O = np.zeros(V.shape)
        for t in range(V.shape[0]):
            alpha = np.exp(G[t][:, None] * A)             # (H, S)
            st = alpha[:, :, None] * st + Bk[t][:, :, None] * V[t][:, None, :]
            O[t] = np.einsum("hs,hsd->hd", Ck[t], st)
        out[sel] = O
        hT[n] = st
    return epilogue(out, v, D, gate), hT


def diag_fwd_unrolled(v, b, c, g, A_log, h0=None, cu_seqlens=None, D=None, gate=None):
    """The unrolled sum of Walkthrough section 5.3.1, evaluated term by term.

    H_t = w(0, t) (.) H_0 + sum_{tau <= t} w(tau, t) (.) (b_tau v_tau^T) with
    w(tau, t) = exp(A * sum_{j = tau+1..t} g_j) per key row (w(t, t) = 1 and
    w(0, t) the product of every decay up to t).  Nothing is carried from one
    t to the next: each output is summed afresh.
    """
    v, b, c, g, A_log, h0 = map(_f64, (v, b, c, g, A_log, h0))
    B, T, H, S, Dv = _dims(v, b, cu_seqlens)
    A = -np.exp(A_log)
    out = np.zeros(v.shape, dtype=np.float64)
    hT = np.zeros((B, H, S, Dv), dtype=np.float64)
    for n, sel in _chains(v, cu_seqlens):
        V, Bk, Ck, G = v[sel], b[sel], c[sel], g[sel]
        L = V.shape[0]
        O = np.zeros(V.shape)
        for h in range(H):
            for t in range(-1, L):
                # decay of the initial state: every token 0..t
                st = np.zeros((S, Dv))
                if h0 is not None:
                    st = np.exp(A[h] * np.sum(G[: t + 1, h]))[:, None] * h0[n, h]
                for tau in range(t + 1):
                    w = np.exp(A[h] * np.sum(G[tau + 1: t + 1, h]))
                    st = st + w[:, None] * np.outer(Bk[tau, h], V[tau, h])
                if t >= 0:
                    O[t, h] = Ck[t, h] @ st
                if t == L - 1:
                    hT[n, h] = st
        out[sel] = O
    return epilogue(out, v, D, gate), hT
