"""Pins for the diagonal-decay additive recurrence: facts that hold
independently of any implementation of it.  They check the FP64 oracle (and,
through the mutant test, show that each plausible mistake breaks at least
one of them).

Every pin takes ``fwd(v, b, c, g, A_log, h0=None, cu=None, D=None,
gate=None) -> (out, hT)`` in float64 and raises ``AssertionError`` when the
fact does not hold.  The recurrence (HyMo "Model Architecture Walkthrough",
section 5.2.1): H_t = exp(g_t A) (.) H_{t-1} + b_t (x) v_t, o_t = c_t^T H_t,
A = -exp(A_log); epilogue (section 5.5 step 6): (o + D_h v) * gate.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand(rng, B, T, H, S, D, h0=False, epi=False):
    v = rng.standard_normal((B, T, H, D))
    b = rng.standard_normal((B, T, H, S)) / np.sqrt(S)
    c = rng.standard_normal((B, T, H, S)) / np.sqrt(S)
    g = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    A_log = rng.uniform(-1.0, 1.5, size=(H, S))
    x = dict(v=v, b=b, c=c, g=g, A_log=A_log)
    if h0:
        x["h0"] = rng.standard_normal((B, H, S, D))
    if epi:
        x["D"] = 1.0 + 0.3 * rng.standard_normal(H)
        x["gate"] = rng.uniform(0.1, 0.9, size=(B, T, H))
    return x


def _close(a, b, tol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"max abs diff {err:.3e} (scale {scale:.3g})"


def pin_hand_example(fwd, rng):
    """The hand-worked two-token example (S=2, D=3, initial state, epilogue)."""
    with open(os.path.join(GOLDEN, "diag_hand_two_tokens.json")) as f:
        gd = json.load(f)
    arr = lambda k: np.array(gd[k], dtype=np.float64)
    g = np.full((1, 2, 1), np.log(2.0))
    out, hT = fwd(arr("v"), arr("b"), arr("c"), g, arr("A_log"), h0=arr("h0"))
    _close(out, arr("out_plain"))
    _close(hT, arr("hT"))
    out, hT = fwd(arr("v"), arr("b"), arr("c"), g, arr("A_log"), h0=arr("h0"),
                  D=arr("Dskip"), gate=arr("gate"))
    _close(out, arr("out"))
    _close(hT, arr("hT"))


def pin_no_memory(fwd, rng):
    """Decay so strong that exp(g A) is exactly 0: each output sees only its
    own token's write, o_t = (c_t . b_t) v_t, and the final state is the last
    write alone (Walkthrough 5.3.2: the fastest heads keep only the current
    step); the epilogue then gives ((c_t . b_t) + D_h) v_t gate_t."""
    x = rand(rng, 2, 9, 3, 5, 4, h0=True)
    x["A_log"] = np.full((3, 5), 30.0)           # A = -1.07e13
    out, hT = fwd(**x)
    cb = np.sum(x["c"] * x["b"], axis=-1)
    _close(out, cb[..., None] * x["v"])
    _close(hT, x["b"][:, -1, :, :, None] * x["v"][:, -1, :, None, :])
    # with the epilogue: ((c_t . b_t) + D_h) v_t * gate_t
    Dk = 1.0 + 0.3 * rng.standard_normal(3)
    gate = rng.uniform(0.1, 0.9, size=(2, 9, 3))
    out, _ = fwd(**x, D=Dk, gate=gate)
    _close(out, ((cb + Dk) * gate)[..., None] * x["v"])


def pin_linear_attention(fwd, rng):
    """With g = 0 nothing decays and the layer is causal linear attention:
    o_t = c_t^T H_0 + sum_{tau <= t} (c_t . b_tau) v_tau, i.e. the masked
    product tril(C B^T) V (Walkthrough 5.2.3 names linear attention as the
    special case without gating)."""
    x = rand(rng, 2, 11, 2, 6, 3, h0=True)
    x["g"] = np.zeros_like(x["g"])
    out, hT = fwd(**x)
    for bb in range(2):
        for h in range(2):
            C, Bk, V = x["c"][bb, :, h], x["b"][bb, :, h], x["v"][bb, :, h]
            H0 = x["h0"][bb, h]
            ref = np.tril(C @ Bk.T) @ V + C @ H0
            _close(out[bb, :, h], ref)
            _close(hT[bb, h], H0 + Bk.T @ V)


def pin_geometric(fwd, rng):
    """S = D = 1, constant decay a = exp(g A), b = c = v = 1: the state is the
    geometric sum h_t = a^(t+1) h_0 + (1 - a^(t+1)) / (1 - a)."""
    T = 23
    gval, A_log = 0.3, np.log(0.7)
    a = np.exp(-gval * np.exp(A_log))
    one = np.ones((1, T, 1, 1))
    h0 = np.full((1, 1, 1, 1), 2.5)
    out, hT = fwd(one, one, one, np.full((1, T, 1), gval), np.full((1, 1), A_log), h0=h0)
    t = np.arange(T)
    ref = a ** (t + 1) * 2.5 + (1 - a ** (t + 1)) / (1 - a)
    _close(out[0, :, 0, 0], ref)
    _close(hT[0, 0, 0, 0], ref[-1])


def pin_rows_decay_independently(fwd, rng):
    """Each key row decays by its own factor: changing A_log of row s leaves
    a read of the other rows (c zero on row s) unchanged, and a read of row s
    alone equals the scalar recurrence of that row."""
    x = rand(rng, 1, 13, 2, 4, 3, h0=True)
    mask = np.array([1.0, 1.0, 0.0, 1.0])
    x["c"] = x["c"] * mask
    out1, hT1 = fwd(**x)
    y = dict(x)
    y["A_log"] = x["A_log"].copy()
    y["A_log"][:, 2] += 1.7
    out2, hT2 = fwd(**y)
    _close(out1, out2)
    _close(np.delete(hT1, 2, axis=2), np.delete(hT2, 2, axis=2))
    # row 2 alone: h_t = exp(g_t A_2) h_{t-1} + b_t[2] v_t
    z = dict(x)
    z["c"] = np.zeros_like(x["c"])
    z["c"][..., 2] = 1.0
    out3, hT3 = fwd(**z)
    for h in range(2):
        A2 = -np.exp(x["A_log"][h, 2])
        st = x["h0"][0, h, 2].copy()
        for t in range(13):
            st = np.exp(x["g"][0, t, h] * A2) * st + x["b"][0, t, h, 2] * x["v"][0, t, h]
            _close(out3[0, t, h], st)
        _close(hT3[0, h, 2], st)


def pin_split_composes(fwd, rng):
    """Running [0, t) and then [t, T) from the first part's final state
    equals one run over [0, T) (the state carries all history)."""
    x = rand(rng, 2, 17, 2, 5, 4, h0=True, epi=True)
    out, hT = fwd(**x)
    cut = 6
    first = {k: (val[:, :cut] if k in ("v", "b", "c", "g", "gate") else val) for k, val in x.items()}
    o1, h1 = fwd(**first)
    second = {k: (val[:, cut:] if k in ("v", "b", "c", "g", "gate") else val) for k, val in x.items()}
    second["h0"] = h1
    o2, h2 = fwd(**second)
    _close(np.concatenate([o1, o2], axis=1), out)
    _close(h2, hT)


def pin_packed_equals_dense(fwd, rng):
    """Packed sequences are independent recurrences: the packed call equals
    separate calls per sequence, including an empty sequence (hT = h0)."""
    lens = [5, 0, 9, 1]
    H, S, D = 2, 3, 4
    parts = [rand(rng, 1, L, H, S, D, epi=True) for L in lens]
    h0 = rng.standard_normal((len(lens), H, S, D))
    A_log = parts[0]["A_log"]
    Dk = parts[0]["D"]
    cat = lambda k: np.concatenate([p[k][0] for p in parts], axis=0)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out, hT = fwd(cat("v"), cat("b"), cat("c"), cat("g"), A_log, h0=h0, cu=cu, D=Dk,
                  gate=cat("gate"))
    for n, p in enumerate(parts):
        o, h = fwd(p["v"], p["b"], p["c"], p["g"], A_log, h0=h0[n:n + 1], D=Dk, gate=p["gate"])
        _close(out[cu[n]:cu[n + 1]], o[0])
        _close(hT[n], h[0])


def pin_linear_in_writes(fwd, rng):
    """Outputs and state are linear in (v, h0) jointly, with b, c, g fixed."""
    x = rand(rng, 1, 12, 2, 4, 5, h0=True, epi=True)
    y = dict(x)
    y["v"] = rng.standard_normal(x["v"].shape)
    y["h0"] = rng.standard_normal(x["h0"].shape)
    z = dict(x)
    z["v"] = 2.0 * x["v"] - 3.0 * y["v"]
    z["h0"] = 2.0 * x["h0"] - 3.0 * y["h0"]
    (ox, hx), (oy, hy), (oz, hz) = fwd(**x), fwd(**y), fwd(**z)
    _close(oz, 2.0 * ox - 3.0 * oy, 1e-11)
    _close(hz, 2.0 * hx - 3.0 * hy, 1e-11)


def pin_causal(fwd, rng):
    """Changing tokens after t changes no output at or before t."""
    x = rand(rng, 1, 15, 2, 4, 3, h0=True, epi=True)
    out, _ = fwd(**x)
    y = {k: (val.copy() if isinstance(val, np.ndarray) else val) for k, val in x.items()}
    for k in ("v", "b", "c", "g", "gate"):
        y[k][:, 8:] = rng.standard_normal(y[k][:, 8:].shape) if k != "g" else 0.5
    out2, _ = fwd(**y)
    _close(out2[:, :8], out[:, :8])
    assert np.max(np.abs(out2[:, 8:] - out[:, 8:])) > 1e-3


def pin_epilogue_identity(fwd, rng):
    """At the block's initialisation (no writes, zero state, D = 1, gate = 1)
    the layer passes v through: o_t = v_t (Walkthrough 5.6)."""
    x = rand(rng, 2, 7, 3, 4, 5)
    x["b"] = np.zeros_like(x["b"])
    out, hT = fwd(**x, D=np.ones(3), gate=np.ones((2, 7, 3)))
    _close(out, x["v"])
    _close(hT, 0.0 * hT)


ALL_PINS = [pin_hand_example, pin_no_memory, pin_linear_attention, pin_geometric,
            pin_rows_decay_independently, pin_split_composes, pin_packed_equals_dense,
            pin_linear_in_writes, pin_causal, pin_epilogue_identity]
