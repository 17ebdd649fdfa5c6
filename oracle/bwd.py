"""Oracle for the gradients of the gated delta rule forward pass (FP64, CPU).

TEST INFRASTRUCTURE ONLY.  Only the tests may import this module; the
product library never does, and this module imports nothing from it.

The forward rule (HyMo "Model Architecture Walkthrough", sections 5.2.1 and
5.2.2), per chain, with the state kept as M = S^T (dk x dv):

    alpha = exp(g_t),  p = M^T k_t,  u = beta_t (v_t - alpha p),
    M_t = alpha M_{t-1} + k_t u^T,   o_t = M_t^T q_t.

The pages train through this layer with a backward pass that runs through
time in reverse (the walkthrough's section 6.5 and the "Optimization
Quartet", sections 3.3-3.4).  :func:`bwd_seq` is that reverse sweep: given
the output gradients do (shape of out) and dhT (shape of hT), it returns
dq, dk, dv, dg, dbeta and dh0 of the scalar <do, out> + <dhT, hT>, by
reverse-mode differentiation of the step above taken one operation at a
time, with every forward state stored (small inputs only):

    Lam  <- Lam + q_t do_t^T                    (o_t = M_t^T q_t)
    dq_t  = M_t do_t
    dalpha = <Lam, M_{t-1}>,  dk_t = Lam u,  du = Lam^T k_t
    dbeta_t = <du, v_t - alpha p>,  dv_t = beta du,  dp = -alpha beta du
    dalpha -= beta <du, p>
    Lam  <- alpha Lam + k_t dp^T,   dk_t += M_{t-1} dp
    dg_t  = alpha dalpha

and dh0 is Lam after the first token.  Layouts are those of the forward
oracle (``oracle.fwd_seq``): dense (B,T,H,.) or packed with ``cu_seqlens``.

:func:`bwd_chunked` evaluates the same gradients by the chunkwise reverse
pass (a derived block algebra, not on the pages), as the brute-force check of
that algebra.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _chains(q, cu_seqlens):
    if cu_seqlens is not None:
        for n in range(len(cu_seqlens) - 1):
            yield n, (slice(int(cu_seqlens[n]), int(cu_seqlens[n + 1])),)
    else:
        for n in range(q.shape[0]):
            yield n, (n,)


def bwd_seq(q, k, v, g, beta, h0=None, cu_seqlens=None, do=None, dhT=None):
    """Reverse sweep.  Returns a dict of float64 arrays dq, dk, dv, dg,
    dbeta, dh0 (dh0 has hT's shape even when h0 is None)."""
    q, k, v, g, beta, h0, do, dhT = map(_f64, (q, k, v, g, beta, h0, do, dhT))
    if cu_seqlens is not None:
        T, H, dk_ = q.shape
        B = len(cu_seqlens) - 1
    else:
        B, T, H, dk_ = q.shape
    dv_ = v.shape[-1]
    if do is None:
        do = np.zeros(v.shape)
    grads = {name: np.zeros(x.shape) for name, x in
             (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    grads["dh0"] = np.zeros((B, H, dk_, dv_))
    for n, sel in _chains(q, cu_seqlens):
        Q, K, V, G, Bt, DO = q[sel], k[sel], v[sel], g[sel], beta[sel], do[sel]
        L = Q.shape[0]
        for h in range(H):
            M = np.zeros((dk_, dv_)) if h0 is None else h0[n, h].copy()
            states = [M]
            us, ps = [], []
            for t in range(L):
                a = np.exp(G[t, h])
                p = M.T @ K[t, h]
                u = Bt[t, h] * (V[t, h] - a * p)
                M = a * M + np.outer(K[t, h], u)
                states.append(M)
                us.append(u)
                ps.append(p)
            Lam = np.zeros((dk_, dv_)) if dhT is None else dhT[n, h].copy()
            dQ, dK, dV = np.zeros((L, dk_)), np.zeros((L, dk_)), np.zeros((L, dv_))
            dG, dB = np.zeros(L), np.zeros(L)
            for t in range(L - 1, -1, -1):
                a = np.exp(G[t, h])
                bt = Bt[t, h]
                kt, qt, vt = K[t, h], Q[t, h], V[t, h]
                Mt, Mp = states[t + 1], states[t]
                u, p = us[t], ps[t]
                Lam = Lam + np.outer(qt, DO[t, h])
                dQ[t] = Mt @ DO[t, h]
                dalpha = np.sum(Lam * Mp)
                dK[t] = Lam @ u
                du = Lam.T @ kt
                dB[t] = du @ (vt - a * p)
                dV[t] = bt * du
                dp = -a * bt * du
                dalpha -= bt * (du @ p)
                Lam = a * Lam + np.outer(kt, dp)
                dK[t] += Mp @ dp
                dG[t] = a * dalpha
            # scatter back into the chain's slices
            gq, gk, gv = grads["dq"][sel], grads["dk"][sel], grads["dv"][sel]
            gg, gb = grads["dg"][sel], grads["dbeta"][sel]
            gq[:, h], gk[:, h], gv[:, h], gg[:, h], gb[:, h] = dQ, dK, dV, dG, dB
            grads["dq"][sel], grads["dk"][sel], grads["dv"][sel] = gq, gk, gv
            grads["dg"][sel], grads["dbeta"][sel] = gg, gb
            grads["dh0"][n, h] = Lam
    return grads


def bwd_chunked(q, k, v, g, beta, h0=None, cu_seqlens=None, do=None, dhT=None, chunk=32):
    """The same gradients by the chunkwise reverse pass, in FP64, as a check
    of that block algebra (the GPU kernels follow it; this function shares no
    code with them).  Per chunk of C tokens with entry state M, exit
    gradient dM', gamma the in-chunk cumulative g, Gam = exp(gamma),
    w = exp(gamma_C - gamma), E_ij = exp(gamma_i - gamma_j):

        A = strict_lower(diag(beta) K K^T . E),  T = (I + A)^-1,
        X = diag(beta)(V - diag(Gam) K M),  U = T X,  P = lower(Q K^T . E),
        dU = P^T dO + diag(w) K dM',  dX = T^T dU,
        dM = Gam_C dM' + Q^T diag(Gam) dO - K^T diag(beta Gam) dX,

    and the token gradients of each chunk from its M, dM', X, U, dU, dX by
    the chain rule through A, E, Gam and w (written out below).  The entry
    states come from a forward pass over the chunks; the exit gradients from
    a backward pass over them starting at dhT.
    """
    q, k, v, g, beta, h0, do, dhT = map(_f64, (q, k, v, g, beta, h0, do, dhT))
    if cu_seqlens is not None:
        T, H, dk_ = q.shape
        B = len(cu_seqlens) - 1
    else:
        B, T, H, dk_ = q.shape
    dv_ = v.shape[-1]
    if do is None:
        do = np.zeros(v.shape)
    grads = {name: np.zeros(x.shape) for name, x in
             (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    grads["dh0"] = np.zeros((B, H, dk_, dv_))

    def chunk_terms(Q, K, G, Bt):
        L = K.shape[0]
        gam = np.cumsum(G)
        Gam = np.exp(gam)
        E = np.exp(gam[:, None] - gam[None, :])
        low = np.tril(np.ones((L, L)), -1)
        lowi = np.tril(np.ones((L, L)))
        KK = K @ K.T
        A = Bt[:, None] * KK * E * low
        Tm = np.linalg.inv(np.eye(L) + A)
        P = (Q @ K.T) * E * lowi
        w = np.exp(gam[-1] - gam)
        return Gam, E, low, lowi, KK, A, Tm, P, w

    for n, sel in _chains(q, cu_seqlens):
        Qa, Ka, Va, Ga, Ba, DOa = q[sel], k[sel], v[sel], g[sel], beta[sel], do[sel]
        L = Qa.shape[0]
        starts = list(range(0, L, chunk))
        for h in range(H):
            cut = [slice(s, min(s + chunk, L)) for s in starts]
            terms = [chunk_terms(Qa[c, h], Ka[c, h], Ga[c, h], Ba[c, h]) for c in cut]
            # forward over chunks: entry states
            M = np.zeros((dk_, dv_)) if h0 is None else h0[n, h].copy()
            Ms = []
            for c, (Gam, E, low, lowi, KK, A, Tm, P, w) in zip(cut, terms):
                Ms.append(M)
                X = Ba[c, h][:, None] * (Va[c, h] - Gam[:, None] * (Ka[c, h] @ M))
                M = Gam[-1] * M + Ka[c, h].T @ (w[:, None] * (Tm @ X))
            # backward over chunks: exit gradients
            D = np.zeros((dk_, dv_)) if dhT is None else dhT[n, h].copy()
            Ds = [None] * len(cut)
            for i in range(len(cut) - 1, -1, -1):
                c = cut[i]
                Gam, E, low, lowi, KK, A, Tm, P, w = terms[i]
                Ds[i] = D
                dU = P.T @ DOa[c, h] + w[:, None] * (Ka[c, h] @ D)
                dX = Tm.T @ dU
                D = (Gam[-1] * D + Qa[c, h].T @ (Gam[:, None] * DOa[c, h])
                     - Ka[c, h].T @ ((Ba[c, h] * Gam)[:, None] * dX))
            grads["dh0"][n, h] = D
            # per-chunk token gradients
            out = {"dq": np.zeros((L, dk_)), "dk": np.zeros((L, dk_)), "dv": np.zeros((L, dv_)),
                   "dg": np.zeros(L), "dbeta": np.zeros(L)}
            for i, c in enumerate(cut):
                Gam, E, low, lowi, KK, A, Tm, P, w = terms[i]
                Qc, Kc, Vc, Bc, DOc = Qa[c, h], Ka[c, h], Va[c, h], Ba[c, h], DOa[c, h]
                M, Dx = Ms[i], Ds[i]
                Y = Kc @ M
                R = Vc - Gam[:, None] * Y
                U = Tm @ (Bc[:, None] * R)
                KD = Kc @ Dx
                dU = P.T @ DOc + w[:, None] * KD
                dX = Tm.T @ dU
                dA = -(dX @ U.T) * low
                dP = (DOc @ U.T) * lowi
                Gm = dA * E * Bc[:, None]
                dPE = dP * E
                Z = dA * A + dP * P * low
                dw = np.sum(U * KD, axis=1)
                dGam = -Bc * np.sum(dX * Y, axis=1) + np.sum(DOc * (Qc @ M), axis=1)
                dGam[-1] += np.sum(M * Dx)
                dgam = Z.sum(1) - Z.sum(0) + dGam * Gam - dw * w
                dgam[-1] += np.sum(dw * w)
                out["dv"][c] = Bc[:, None] * dX
                out["dbeta"][c] = np.sum(dX * R, axis=1) + np.sum(dA * KK * E, axis=1)
                out["dq"][c] = Gam[:, None] * (DOc @ M.T) + dPE @ Kc
                out["dk"][c] = (-((Bc * Gam)[:, None] * dX) @ M.T + Gm @ Kc + Gm.T @ Kc
                                + dPE.T @ Qc + w[:, None] * (U @ Dx.T))
                out["dg"][c] = np.cumsum(dgam[::-1])[::-1]
            for name in ("dq", "dk", "dv", "dg", "dbeta"):
                tgt = grads[name][sel]
                tgt[:, h] = out[name]
                grads[name][sel] = tgt
    return grads
