"""Oracle for the gated delta rule forward pass (FP64, CPU).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package; the product library
never does, and this package imports nothing from it.

Three independent evaluations of the same function, all in float64:

* :func:`fwd_seq` -- the C sequential oracle (``gdn_oracle.c``), threaded over
  independent chains, strictly sequential in t.  State kept as M = S^T.
* :func:`fwd_matrix` -- NumPy, the rule written literally as matrices in the
  S orientation: ``S <- alpha S (I - beta k k^T) + beta v k^T``, ``o = S q``.
* :func:`fwd_chunked` -- NumPy, the chunkwise-parallel form with an explicit
  triangular solve, the brute-force check of the block algebra the GPU kernel
  uses.

The rule is the delta rule of HyMo "Model Architecture Walkthrough"
section 5.2.2 (change = rate x (target - prediction) x input) with the
per-head scalar decay alpha_t = exp(g_t) of sections 5.2.1 and 5.3.1; the
read o_t = S_t q_t takes the state after the write (section 5.2.1 reads
H_t).  Keys/queries are passed as they are stored (bf16 or fp32 values,
upcast exactly); no output scale is applied.

Layouts (row-major): dense q,k (B,T,H,dk), v,out (B,T,H,dv), g,beta (B,T,H);
packed (``cu_seqlens`` given): the same without B.  h0/hT (B,H,dk,dv) with
hT[b,h,i,j] = S[j,i] (i over dk, j over dv).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
# GDN_ORACLE_LIB names another build of the C oracle (the tests use it to
# run the pins against an AddressSanitizer/UBSan build).
_LIB = os.environ.get("GDN_ORACLE_LIB") or os.path.join(_HERE, "libgdn_oracle.so")
_lib = None
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                  "-fno-sanitize-recover=undefined"]


def build(force: bool = True, out: Optional[str] = None, sanitize: bool = False) -> str:
    """Compile the C oracle with gcc into ``oracle/libgdn_oracle.so`` (or
    ``out``); ``sanitize`` instruments it with AddressSanitizer and UBSan."""
    global _lib
    target = out or _LIB
    if force or not os.path.exists(target):
        tmp = target + ".tmp"
        flags = ["-O1", "-g"] + SANITIZE_FLAGS if sanitize else ["-O2"]
        subprocess.check_call(["gcc", *flags, "-std=c99", "-fPIC", "-shared",
                               "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, target)
        if target == _LIB:
            _lib = None
    return target


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.gdn_oracle_fwd.restype = ctypes.c_int
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.gdn_oracle_fwd.argtypes = [P, P, P, P, P, P, P, P, P,
                                       I, I, I, I, I, P, I, I]
        _lib = lib
    return _lib


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _dims(q, v, cu_seqlens, h0):
    if cu_seqlens is not None:
        T, H, dk = q.shape
        B = len(cu_seqlens) - 1
    else:
        B, T, H, dk = q.shape
    dv = v.shape[-1]
    return B, T, H, dk, dv


def fwd_seq(q, k, v, g, beta, h0=None, cu_seqlens=None,
            chains: Optional[Sequence[int]] = None, nthreads: Optional[int] = None,
            out=None, hT=None):
    """C sequential oracle.  Returns (out, hT) as float64 arrays.

    ``chains`` restricts the work to chain ids ``b*H + h`` (other chains'
    outputs are zero, or left as in the passed ``out``/``hT``).
    """
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    B, T, H, dk, dv = _dims(q, v, cu, h0)
    if out is None:
        out = np.zeros(v.shape, dtype=np.float64)
    if hT is None:
        hT = np.zeros((B, H, dk, dv), dtype=np.float64)
    ch = None if chains is None else np.ascontiguousarray(chains, dtype=np.int32)
    nthreads = nthreads or (os.cpu_count() or 1)
    rc = _load().gdn_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(h0), _ptr(cu), _ptr(out), _ptr(hT),
                                B, T, H, dk, dv, _ptr(ch),
                                0 if ch is None else len(ch), int(nthreads))
    if rc != 0:
        raise ValueError("gdn_oracle_fwd: invalid arguments")
    return out, hT


def _chains(q, v, cu_seqlens):
    """Yield (b, h, index tuple selecting the chain's tokens)."""
    if cu_seqlens is not None:
        T, H, _ = q.shape
        for b in range(len(cu_seqlens) - 1):
            s, e = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
            for h in range(H):
                yield b, h, (slice(s, e), h)
    else:
        B, T, H, _ = q.shape
        for b in range(B):
            for h in range(H):
                yield b, h, (b, slice(0, T), h)


def fwd_matrix(q, k, v, g, beta, h0=None, cu_seqlens=None):
    """The rule as literal matrix products in the S (dv x dk) orientation.

    Per step: ``S <- alpha S (I - beta k k^T) + beta v k^T`` then
    ``o = S q`` (HyMo "Model Architecture Walkthrough", sections 5.2.1-5.2.2
    for the delta-rule write and the read after the write).  Pure-Python loop
    over tokens: small inputs only.
    """
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    B, T, H, dk, dv = _dims(q, v, cu_seqlens, h0)
    out = np.zeros(v.shape, dtype=np.float64)
    hT = np.zeros((B, H, dk, dv), dtype=np.float64)
    I = np.eye(dk)
    for b, h, sel in _chains(q, v, cu_seqlens):
        S = np.zeros((dv, dk)) if h0 is None else h0[b, h].T.copy()
        Q, K, V, G, Bt = q[sel], k[sel], v[sel], g[sel], beta[sel]
        O = out[sel]
        for t in range(K.shape[0]):
            kt = K[t][:, None]
            S = np.exp(G[t]) * S @ (I - Bt[t] * (kt @ kt.T)) + Bt[t] * (V[t][:, None] @ kt.T)
            O[t] = S @ Q[t]
        out[sel] = O
        hT[b, h] = S.T
    return out, hT


def fwd_chunked(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk: int = 64):
    """Chunkwise-parallel evaluation with an explicit triangular solve.

    The pages' kernel cuts each sequence into chunks (default 64), works on a
    chunk in parallel and carries the state across chunks in series ("v1.0
    Architecture & Design Spec", section 2.3; "Optimization Quartet",
    section 3.2).  The pages print no formulas for it; the block algebra
    below follows from unrolling the rule over one chunk.

    For a chunk with rows r = 1..C (relative to the chunk start), state M at
    chunk entry (M = S^T, dk x dv), gamma = cumsum(g) inside the chunk and
    Gam = exp(gamma):

      A    = strictly-lower part of  diag(beta) (K K^T) * exp(gamma_i - gamma_j)
      Tinv = (I + A)^{-1}
      W    = Tinv diag(beta * Gam) K            (C x dk)
      Uh   = Tinv diag(beta) V                  (C x dv)
      U    = Uh - W M                           (the per-token corrected writes)
      O    = diag(Gam) Q M + ((Q K^T) * exp(gamma_i - gamma_j), j <= i) U
      M   <- Gam_C M + (diag(exp(gamma_C - gamma)) K)^T U

    A chunk that runs past the end of a sequence is simply shorter.  This is
    a plain FP64 evaluation with ``numpy.linalg.solve`` for the inverse.
    """
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    B, T, H, dk, dv = _dims(q, v, cu_seqlens, h0)
    out = np.zeros(v.shape, dtype=np.float64)
    hT = np.zeros((B, H, dk, dv), dtype=np.float64)
    for b, h, sel in _chains(q, v, cu_seqlens):
        M = np.zeros((dk, dv)) if h0 is None else h0[b, h].copy()
        Q, K, V, G, Bt = q[sel], k[sel], v[sel], g[sel], beta[sel]
        O = np.zeros(V.shape)
        L = K.shape[0]
        for s in range(0, L, chunk):
            e = min(s + chunk, L)
            Qc, Kc, Vc, bc = Q[s:e], K[s:e], V[s:e], Bt[s:e]
            gam = np.cumsum(G[s:e])
            n = e - s
            diff = gam[:, None] - gam[None, :]
            lower_incl = np.tril(np.ones((n, n), dtype=bool))
            D = np.where(lower_incl, np.exp(np.where(lower_incl, diff, 0.0)), 0.0)
            A = np.tril(bc[:, None] * (Kc @ Kc.T) * D, k=-1)
            Tinv = np.linalg.solve(np.eye(n) + A, np.eye(n))
            Gam = np.exp(gam)
            W = Tinv @ ((bc * Gam)[:, None] * Kc)
            Uh = Tinv @ (bc[:, None] * Vc)
            U = Uh - W @ M
            O[s:e] = Gam[:, None] * (Qc @ M) + ((Qc @ Kc.T) * D) @ U
            M = Gam[-1] * M + (np.exp(gam[-1] - gam)[:, None] * Kc).T @ U
        out[sel] = O
        hT[b, h] = M
    return out, hT


def rel_err(x, ref) -> float:
    """Infinity-norm relative error max|x - ref| / max|ref| (0/0 -> 0)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(x - ref)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
