"""Pins: facts about the gated delta rule that hold independently of any
implementation of it, used to check the FP64 oracle (and, through the mutant
test, to show that each plausible mistake in an implementation breaks at
least one of them).

Every pin takes ``fwd(q, k, v, g, beta, h0=None, cu_seqlens=None) ->
(out, hT)`` in float64 and raises ``AssertionError`` when the fact does not
hold.  The rule (HyMo "Model Architecture Walkthrough", sections 5.2.1 and
5.2.2): S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
o_t = S_t q_t, alpha_t = exp(g_t), hT[b,h] = S_T^T.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand(rng, B, T, H, dk, dv, h0=False, g_scale=1.0):
    q = _unit(rng.standard_normal((B, T, H, dk)))
    k = _unit(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    g = -np.logaddexp(0.0, rng.standard_normal((B, T, H))) * g_scale
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    M0 = rng.standard_normal((B, H, dk, dv)) * 0.5 if h0 else None
    return q, k, v, g, beta, M0


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol:.1e} * {scale:.3g}"


# ------------------------------------------------------------------ pins --

def pin_golden(fwd, rng=None):
    """Hand-worked examples under tests/golden (derivations in each file)."""
    for name in sorted(os.listdir(GOLDEN)):
        # diag_*.json belong to the diagonal-decay form (tests/pins_diag.py)
        if not name.endswith(".json") or name.startswith("diag_"):
            continue
        with open(os.path.join(GOLDEN, name)) as f:
            d = json.load(f)
        q, k, v = (np.array(d[x], dtype=np.float64) for x in ("q", "k", "v"))
        g = np.log(np.array(d["alpha"], dtype=np.float64))
        beta = np.array(d["beta"], dtype=np.float64)
        h0 = None if d["h0"] is None else np.array(d["h0"], dtype=np.float64)
        cu = d.get("cu_seqlens")
        cu = None if cu is None else np.array(cu, dtype=np.int32)
        out, hT = fwd(q, k, v, g, beta, h0, cu)
        _close(out, np.array(d["out"]), 1e-12, f"{name} out")
        _close(hT, np.array(d["hT"]), 1e-12, f"{name} hT")


def pin_single_step(fwd, rng):
    """T = 1.  From a zero state the write is beta k v^T, so o = beta (k.q) v
    and hT = beta k v^T.  From M0 the state after one step, in the hT
    orientation, is alpha (I - beta k k^T) M0 + beta k v^T."""
    for dk, dv in ((5, 3), (3, 5), (4, 4)):
        q, k, v, g, beta, _ = _rand(rng, 2, 1, 3, dk, dv)
        out, hT = fwd(q, k, v, g, beta, None, None)
        kq = np.sum(k * q, axis=-1)                      # (B,1,H)
        _close(out, (beta * kq)[..., None] * v, 1e-13, "T=1 out, zero state")
        want = beta[:, 0, :, None, None] * k[:, 0, :, :, None] * v[:, 0, :, None, :]
        _close(hT, want, 1e-13, "T=1 hT, zero state")
        M0 = rng.standard_normal((2, 3, dk, dv))
        out, hT = fwd(q, k, v, g, beta, M0, None)
        a = np.exp(g[:, 0])[..., None, None]
        b = beta[:, 0][..., None, None]
        kk = k[:, 0, :, :, None] * k[:, 0, :, None, :]
        want = a * (M0 - b * kk @ M0) + b * k[:, 0, :, :, None] * v[:, 0, :, None, :]
        _close(hT, want, 1e-13, "T=1 hT from M0")
        _close(out[:, 0], np.einsum("bhij,bhi->bhj", want, q[:, 0]), 1e-13, "T=1 out from M0")


def pin_pure_decay(fwd, rng):
    """beta = 0: nothing is written, the state only decays:
    hT = exp(sum g) h0 and o_t = exp(sum_{j<=t} g_j) h0^T q_t."""
    q, k, v, g, beta, M0 = _rand(rng, 2, 23, 2, 6, 4, h0=True)
    beta = np.zeros_like(beta)
    out, hT = fwd(q, k, v, g, beta, M0, None)
    G = np.cumsum(g, axis=1)                                  # (B,T,H)
    _close(hT, np.exp(G[:, -1])[..., None, None] * M0, 1e-13, "beta=0 hT")
    want = np.exp(G)[..., None] * np.einsum("bhij,bthi->bthj", M0, q)
    _close(out, want, 1e-13, "beta=0 out")


def pin_orthonormal_recall(fwd, rng):
    """alpha = 1, beta = 1, keys orthonormal: each write stores v_i exactly
    along k_i and leaves the other key directions alone, so hT^T k_i = v_i
    for every i, hT = sum_i k_i v_i^T from a zero state, and a read with
    q_t = k_s (s <= t) returns v_s."""
    dk, dv, T = 8, 5, 6
    for use_h0 in (False, True):
        Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        k = Qm[:T][None, :, None, :]                     # (1,T,1,dk), orthonormal rows
        v = rng.standard_normal((1, T, 1, dv))
        src = np.array([min(t, int(s)) for t, s in enumerate(rng.integers(0, T, size=T))])
        q = k[:, src]
        g = np.zeros((1, T, 1))
        beta = np.ones((1, T, 1))
        M0 = rng.standard_normal((1, 1, dk, dv)) if use_h0 else None
        out, hT = fwd(q, k, v, g, beta, M0, None)
        _close(np.einsum("ij,ti->tj", hT[0, 0], k[0, :, 0]), v[0, :, 0], 1e-12, "recall hT^T k = v")
        _close(out[0, :, 0], v[0, src, 0], 1e-12, "recall o_t = v_src")
        if not use_h0:
            _close(hT[0, 0], k[0, :, 0].T @ v[0, :, 0], 1e-12, "recall hT = sum k v^T")


def pin_exact_write(fwd, rng):
    """beta = 1 and |k| = 1: any alpha, any initial state, the step makes the
    state map k_t to v_t exactly, so reading with q_t = k_t returns v_t."""
    q, k, v, g, beta, M0 = _rand(rng, 2, 17, 3, 7, 5, h0=True)
    beta = np.ones_like(beta)
    out, _ = fwd(k, k, v, g, beta, M0, None)
    _close(out, v, 1e-12, "beta=1 exact write")


def pin_constant_input(fwd, rng):
    """Constant unit key k (used as the query too), value v, alpha, beta from
    a zero state: along k the state obeys x_t = alpha (1 - beta) x_{t-1} +
    beta v, so o_t = beta v (1 - r^t) / (1 - r) with r = alpha (1 - beta)."""
    dk, dv, T = 6, 4, 40
    k = _unit(rng.standard_normal(dk))
    v = rng.standard_normal(dv)
    for alpha, b in ((0.9, 0.3), (0.5, 0.8), (1.0, 0.25)):
        K = np.broadcast_to(k, (1, T, 1, dk)).copy()
        V = np.broadcast_to(v, (1, T, 1, dv)).copy()
        g = np.full((1, T, 1), np.log(alpha))
        beta = np.full((1, T, 1), b)
        out, hT = fwd(K, K, V, g, beta, None, None)
        r = alpha * (1 - b)
        t = np.arange(1, T + 1)
        want = b * (1 - r ** t)[:, None] / (1 - r) * v[None, :]
        _close(out[0, :, 0], want, 1e-12, f"geometric series alpha={alpha} beta={b}")
        _close(hT[0, 0], np.outer(k, want[-1]), 1e-12, "geometric series hT")


def pin_linearity(fwd, rng):
    """For fixed q, k, g, beta the map (v, h0) -> (o, hT) is linear."""
    q, k, v1, g, beta, M1 = _rand(rng, 1, 19, 2, 5, 4, h0=True)
    v2 = rng.standard_normal(v1.shape)
    M2 = rng.standard_normal(M1.shape)
    a, b = 0.7, -1.9
    o1, h1 = fwd(q, k, v1, g, beta, M1, None)
    o2, h2 = fwd(q, k, v2, g, beta, M2, None)
    o3, h3 = fwd(q, k, a * v1 + b * v2, g, beta, a * M1 + b * M2, None)
    _close(o3, a * o1 + b * o2, 1e-12, "linearity out")
    _close(h3, a * h1 + b * h2, 1e-12, "linearity hT")


def pin_causality(fwd, rng):
    """Inputs at positions after t cannot change o_1..o_t (exactly)."""
    q, k, v, g, beta, M0 = _rand(rng, 1, 21, 2, 4, 3, h0=True)
    out, _ = fwd(q, k, v, g, beta, M0, None)
    t = 9
    q2, k2, v2, g2, b2 = (x.copy() for x in (q, k, v, g, beta))
    for x in (q2, k2, v2):
        x[:, t + 1:] = rng.standard_normal(x[:, t + 1:].shape)
    g2[:, t + 1:] = -rng.random(g2[:, t + 1:].shape)
    b2[:, t + 1:] = rng.random(b2[:, t + 1:].shape)
    out2, _ = fwd(q2, k2, v2, g2, b2, M0, None)
    assert np.array_equal(out[:, : t + 1], out2[:, : t + 1]), "causality: o_<=t changed"
    assert not np.allclose(out[:, t + 1:], out2[:, t + 1:]), "causality: later outputs ignore inputs"


def pin_split(fwd, rng):
    """Running tokens [0, t) then [t, T) from the first part's final state
    equals one run over [0, T)."""
    q, k, v, g, beta, M0 = _rand(rng, 2, 29, 2, 5, 6, h0=True)
    out, hT = fwd(q, k, v, g, beta, M0, None)
    for t in (1, 11, 16):
        oa, ha = fwd(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], M0, None)
        ob, hb = fwd(q[:, t:], k[:, t:], v[:, t:], g[:, t:], beta[:, t:], ha, None)
        _close(np.concatenate([oa, ob], axis=1), out, 1e-12, f"split at {t} out")
        _close(hb, hT, 1e-12, f"split at {t} hT")


def pin_packed(fwd, rng):
    """Each sequence of a packed batch equals that sequence run alone (same
    h0), including empty sequences (hT = h0) and single tokens."""
    lens = [7, 0, 1, 12, 5]
    H, dk, dv = 2, 4, 3
    N = sum(lens)
    q, k, v, g, beta, _ = _rand(rng, 1, N, H, dk, dv)
    q, k, v, g, beta = (x[0] for x in (q, k, v, g, beta))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    M0 = rng.standard_normal((len(lens), H, dk, dv))
    out, hT = fwd(q, k, v, g, beta, M0, cu)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        o1, h1 = fwd(q[None, s:e], k[None, s:e], v[None, s:e], g[None, s:e],
                     beta[None, s:e], M0[n:n + 1], None)
        _close(out[s:e], o1[0], 1e-13, f"packed seq {n} out")
        _close(hT[n], h1[0], 1e-13, f"packed seq {n} hT")
        if e == s:
            _close(hT[n], M0[n], 0.0, "empty sequence keeps h0")


def pin_stability(fwd, rng):
    """For |k| = 1 and 0 <= beta <= 1 the step is a decay times a
    contraction plus a write of size beta |v|:
    |M_t|_2 <= alpha_t |M_{t-1}|_2 + beta_t |v_t|."""
    q, k, v, g, beta, M0 = _rand(rng, 1, 12, 1, 5, 4, h0=True)
    prev = np.linalg.norm(M0[0, 0], 2)
    for t in range(12):
        _, hT = fwd(q[:, : t + 1], k[:, : t + 1], v[:, : t + 1], g[:, : t + 1],
                    beta[:, : t + 1], M0, None)
        cur = np.linalg.norm(hT[0, 0], 2)
        bound = np.exp(g[0, t, 0]) * prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert cur <= bound * (1 + 1e-12), f"stability bound broken at t={t}"
        prev = cur


ALL_PINS = [pin_golden, pin_single_step, pin_pure_decay, pin_orthonormal_recall,
            pin_exact_write, pin_constant_input, pin_linearity, pin_causality,
            pin_split, pin_packed, pin_stability]
