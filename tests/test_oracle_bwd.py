"""The FP64 backward oracle against what the gradient is by definition
(central finite differences of the pinned forward oracle), an adjoint
identity, closed forms of the no-write case, and planted mistakes."""
import numpy as np
import pytest

import oracle
from oracle import bwd as obwd


def _inputs(rng, B=2, T=5, H=2, dk=3, dv=4, packed=False):
    def unit(x):
        return x / np.linalg.norm(x, axis=-1, keepdims=True)
    lead = (T,) if packed else (B, T)
    x = dict(q=unit(rng.standard_normal(lead + (H, dk))), k=unit(rng.standard_normal(lead + (H, dk))),
             v=rng.standard_normal(lead + (H, dv)),
             g=-np.logaddexp(0.0, rng.standard_normal(lead + (H,)) - 1.0),
             beta=1.0 / (1.0 + np.exp(-rng.standard_normal(lead + (H,)))),
             h0=rng.standard_normal((B, H, dk, dv)))
    return x


def _loss(x, do, dhT, cu=None):
    out, hT = oracle.fwd_matrix(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], cu)
    return float(np.sum(out * do) + np.sum(hT * dhT))


def _fd_check(bwd, rng, packed=False, tol=1e-6):
    cu = np.array([0, 2, 2, 5], dtype=np.int32) if packed else None
    x = _inputs(rng, B=3 if packed else 2, T=5, packed=packed)
    out, hT = oracle.fwd_matrix(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], cu)
    do, dhT = rng.standard_normal(out.shape), rng.standard_normal(hT.shape)
    grads = bwd(**x, cu_seqlens=cu, do=do, dhT=dhT)
    eps = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                        ("h0", "dh0")):
        num = np.zeros(x[name].shape)
        for i in np.ndindex(x[name].shape):
            y = {kk: vv.copy() for kk, vv in x.items()}
            y[name][i] += eps
            lp = _loss(y, do, dhT, cu)
            y[name][i] -= 2 * eps
            lm = _loss(y, do, dhT, cu)
            num[i] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(num - grads[gname])) / max(1.0, np.max(np.abs(num)))
        assert err < tol, f"{gname}: {err:.2e}"


def test_matches_finite_differences_dense():
    _fd_check(obwd.bwd_seq, np.random.default_rng(50))


def test_matches_finite_differences_packed_with_empty_sequence():
    _fd_check(obwd.bwd_seq, np.random.default_rng(51), packed=True)


def test_adjoint_identity():
    """(out, hT) is jointly linear in (v, h0), so <do,out> + <dhT,hT> =
    <dv,v> + <dh0,h0> for any do, dhT (Euler's identity for a linear map)."""
    rng = np.random.default_rng(52)
    x = _inputs(rng, B=2, T=9, H=3, dk=4, dv=5)
    out, hT = oracle.fwd_matrix(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    do, dhT = rng.standard_normal(out.shape), rng.standard_normal(hT.shape)
    gr = obwd.bwd_seq(**x, do=do, dhT=dhT)
    lhs = np.sum(do * out) + np.sum(dhT * hT)
    rhs = np.sum(gr["dv"] * x["v"]) + np.sum(gr["dh0"] * x["h0"])
    assert abs(lhs - rhs) < 1e-11 * max(1.0, abs(lhs))


def test_no_write_closed_forms():
    """beta = 0: nothing is written, o_t = e^{gamma_t} h0^T q_t and hT =
    e^{gamma_T} h0 (gamma = cumsum g).  Then dq_t = e^{gamma_t} h0 do_t,
    dh0 = sum_t e^{gamma_t} q_t do_t^T + e^{gamma_T} dhT, dv = 0, dk = 0,
    dg_j = sum_{t>=j} e^{gamma_t} q_t^T h0 do_t + e^{gamma_T} <dhT, h0>."""
    rng = np.random.default_rng(53)
    x = _inputs(rng, B=1, T=6, H=1, dk=3, dv=2)
    x["beta"] = np.zeros_like(x["beta"])
    out, hT = oracle.fwd_matrix(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    do, dhT = rng.standard_normal(out.shape), rng.standard_normal(hT.shape)
    gr = obwd.bwd_seq(**x, do=do, dhT=dhT)
    Q, G, H0, DO = x["q"][0, :, 0], x["g"][0, :, 0], x["h0"][0, 0], do[0, :, 0]
    gam = np.cumsum(G)
    e = np.exp(gam)
    np.testing.assert_allclose(gr["dq"][0, :, 0], e[:, None] * (DO @ H0.T), rtol=1e-12, atol=1e-14)
    ref_dh0 = (e[:, None, None] * Q[:, :, None] * DO[:, None, :]).sum(0) + e[-1] * dhT[0, 0]
    np.testing.assert_allclose(gr["dh0"][0, 0], ref_dh0, rtol=1e-12, atol=1e-14)
    assert np.all(gr["dv"] == 0) and np.all(gr["dk"] == 0)
    per_t = e * np.einsum("ti,ij,tj->t", Q, H0, DO)
    ref_dg = np.cumsum(per_t[::-1])[::-1] + e[-1] * np.sum(dhT[0, 0] * H0)
    np.testing.assert_allclose(gr["dg"][0, :, 0], ref_dg, rtol=1e-12, atol=1e-14)


def test_packed_equals_per_sequence():
    rng = np.random.default_rng(54)
    lens = [3, 0, 4]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = _inputs(rng, B=3, T=7, H=2, dk=3, dv=2, packed=True)
    out, hT = oracle.fwd_matrix(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], cu)
    do, dhT = rng.standard_normal(out.shape), rng.standard_normal(hT.shape)
    gr = obwd.bwd_seq(**x, cu_seqlens=cu, do=do, dhT=dhT)
    for n in range(3):
        s, e = cu[n], cu[n + 1]
        one = {kk: (vv[s:e][None] if kk != "h0" else vv[n:n + 1]) for kk, vv in x.items()}
        g1 = obwd.bwd_seq(**one, do=do[s:e][None], dhT=dhT[n:n + 1])
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            np.testing.assert_allclose(gr[name][s:e], g1[name][0], rtol=0, atol=0)
        np.testing.assert_allclose(gr["dh0"][n], g1["dh0"][0], rtol=0, atol=0)


# ------------------------------------------------------- planted mistakes ---

def _mutant(kind):
    """A copy of the reverse sweep with one planted mistake (CPU only)."""
    def bwd(q, k, v, g, beta, h0=None, cu_seqlens=None, do=None, dhT=None):
        B = h0.shape[0]
        qq, kk, vv, gg, bb = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
        spans = ([(int(cu_seqlens[i]), int(cu_seqlens[i + 1])) for i in range(len(cu_seqlens) - 1)]
                 if cu_seqlens is not None else [(0, q.shape[1])] * B)
        sel = (lambda n, t: (t,)) if cu_seqlens is not None else (lambda n, t: (n, t))
        H, dk_, dv_ = q.shape[-2], q.shape[-1], v.shape[-1]
        out = {nm: np.zeros(np.shape(a)) for nm, a in (("dq", q), ("dk", k), ("dv", v), ("dg", g),
                                                        ("dbeta", beta))}
        out["dh0"] = np.zeros((B, H, dk_, dv_))
        for n, (s0, e0) in enumerate(spans):
            for h in range(H):
                M = np.array(h0[n, h], dtype=np.float64)
                st, us, ps = [M], [], []
                for t in range(s0, e0):
                    i = sel(n, t)
                    a = np.exp(gg[i][h])
                    p = M.T @ kk[i][h]
                    u = bb[i][h] * (vv[i][h] - a * p)
                    M = a * M + np.outer(kk[i][h], u)
                    st.append(M); us.append(u); ps.append(p)
                Lam = np.array(dhT[n, h], dtype=np.float64)
                for j in range(e0 - s0 - 1, -1, -1):
                    i = sel(n, s0 + j)
                    a, bt = np.exp(gg[i][h]), bb[i][h]
                    kt, qt, vt = kk[i][h], qq[i][h], vv[i][h]
                    Mt, Mp, u, p = st[j + 1], st[j], us[j], ps[j]
                    Lam = Lam + np.outer(qt, do[i][h])
                    out["dq"][i + (h,)] = (Mp if kind == "dq_old_state" else Mt) @ do[i][h]
                    dalpha = np.sum(Lam * Mp)
                    dkt = Lam @ u
                    du = Lam.T @ kt
                    out["dbeta"][i + (h,)] = du @ (vt - (0 if kind == "dbeta_no_prediction" else a) * p)
                    out["dv"][i + (h,)] = bt * du
                    dp = (1 if kind == "dp_sign" else -1) * a * bt * du
                    if kind != "dalpha_no_prediction":
                        dalpha -= bt * (du @ p)
                    Lam = (Lam if kind == "no_decay_on_adjoint" else a * Lam) + \
                        (0 if kind == "no_erase_adjoint" else np.outer(kt, dp))
                    out["dk"][i + (h,)] = dkt + Mp @ dp
                    out["dg"][i + (h,)] = (1.0 if kind == "dg_missing_alpha" else a) * dalpha
                out["dh0"][n, h] = Lam
        return out
    return bwd


MUTATIONS = ["dq_old_state", "dbeta_no_prediction", "dp_sign", "dalpha_no_prediction",
             "no_decay_on_adjoint", "no_erase_adjoint", "dg_missing_alpha"]


def test_unmutated_copy_passes():
    _fd_check(_mutant("none"), np.random.default_rng(50))


@pytest.mark.parametrize("kind", MUTATIONS)
def test_mutant_is_caught(kind):
    with pytest.raises(AssertionError):
        _fd_check(_mutant(kind), np.random.default_rng(50))


@pytest.mark.parametrize("chunk", [1, 4, 32, 64])
@pytest.mark.parametrize("packed", [False, True])
def test_chunked_form_equals_reverse_sweep(chunk, packed):
    """The chunkwise reverse pass (the block algebra the GPU kernels follow)
    gives the reverse sweep's gradients to rounding, for chunk lengths that
    do and do not divide the sequences, with a nonzero h0 and dhT; the
    packed case includes an empty and a one-token sequence."""
    rng = np.random.default_rng(40 + chunk + (100 if packed else 0))
    cu = np.array([0, 37, 37, 38, 90], dtype=np.int32) if packed else None
    x = _inputs(rng, B=4 if packed else 2, T=90 if packed else 45, H=2, dk=5, dv=4, packed=packed)
    out, hT = oracle.fwd_matrix(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], cu)
    do, dhT = rng.standard_normal(out.shape), rng.standard_normal(hT.shape)
    a = obwd.bwd_seq(**x, cu_seqlens=cu, do=do, dhT=dhT)
    b = obwd.bwd_chunked(**x, cu_seqlens=cu, do=do, dhT=dhT, chunk=chunk)
    for name in a:
        err = float(np.max(np.abs(a[name] - b[name])) / max(np.max(np.abs(a[name])), 1e-300))
        assert err < 1e-12, (name, err)


def test_chunked_form_strong_decay_and_no_state():
    """g = -30 (every exponential factor between tokens underflows) and no
    h0, no dhT: the chunked form still matches, element by element relative
    to each gradient's own scale."""
    rng = np.random.default_rng(77)
    x = _inputs(rng, B=1, T=40, H=1, dk=4, dv=3)
    x["g"] = np.full_like(x["g"], -30.0)
    x["h0"] = None
    do = rng.standard_normal(x["v"].shape)
    a = obwd.bwd_seq(**x, do=do)
    b = obwd.bwd_chunked(**x, do=do, chunk=16)
    for name in a:
        scale = max(np.max(np.abs(a[name])), 1e-300)
        assert np.max(np.abs(a[name] - b[name])) <= 1e-10 * scale, name
