"""The FP64 oracle of the diagonal-decay additive recurrence against facts
the recurrence fixes (hand-worked example, closed forms, special cases,
invariants), its two evaluations against each other, and planted mistakes
(in this file's own copy of the token loop, on the CPU) against the pins."""
import numpy as np
import pytest

from oracle import diag as odiag
from pins_diag import ALL_PINS, rand

import synth.diag as sd


def _seq(v, b, c, g, A_log, h0=None, cu=None, D=None, gate=None):
    return odiag.diag_fwd_seq(v, b, c, g, A_log, h0, cu, D, gate)


def _unrolled(v, b, c, g, A_log, h0=None, cu=None, D=None, gate=None):
    return odiag.diag_fwd_unrolled(v, b, c, g, A_log, h0, cu, D, gate)


IMPLS = {"token_loop": _seq, "unrolled_sum": _unrolled}


@pytest.mark.parametrize("impl", list(IMPLS))
@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(impl, pin):
    pin(IMPLS[impl], np.random.default_rng(4321))


@pytest.mark.parametrize("h0,epi,packed", [(False, False, False), (True, True, False),
                                           (True, True, True)])
def test_loop_equals_unrolled(h0, epi, packed):
    rng = np.random.default_rng(7)
    if packed:
        lens = [4, 0, 7, 3]
        x = rand(rng, 1, sum(lens), 2, 5, 3, epi=epi)
        x = {k: (val[0] if k in ("v", "b", "c", "g", "gate") else val) for k, val in x.items()}
        x["h0"] = rng.standard_normal((len(lens), 2, 5, 3))
        x["cu"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    else:
        x = rand(rng, 2, 9, 2, 5, 3, h0=h0, epi=epi)
    o1, h1 = _seq(**x)
    o2, h2 = _unrolled(**x)
    assert np.max(np.abs(o1 - o2)) < 1e-12 * max(1, np.max(np.abs(o2)))
    assert np.max(np.abs(h1 - h2)) < 1e-12 * max(1, np.max(np.abs(h2)))


def test_synth_workload_shapes():
    inp = sd.generate(sd.WORKLOADS["diag_tiny"])
    wl = inp.wl
    assert inp.v.shape == (wl.B, wl.T, wl.H, wl.D)
    assert inp.b.shape == inp.c.shape == (wl.B, wl.T, wl.H, wl.S)
    assert inp.g.shape == inp.gate.shape == (wl.B, wl.T, wl.H)
    assert inp.A_log.shape == (wl.H, wl.S) and inp.Dskip.shape == (wl.H,)
    assert np.all(inp.g > 0) and np.all(inp.g < 1)
    assert inp.h0.shape == (wl.B, wl.H, wl.S, wl.D)


# ------------------------------------------------------- planted mistakes ---

def _mutant(mutation):
    def fwd(v, b, c, g, A_log, h0=None, cu=None, D=None, gate=None):
        v, b, c, g, A_log = (np.asarray(x, dtype=np.float64) for x in (v, b, c, g, A_log))
        if cu is not None:
            spans = [(int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
            sel = lambda n, t: (t,)
        else:
            spans = [(0, v.shape[1])] * v.shape[0]
            sel = lambda n, t: (n, t)
        H, S, Dv = b.shape[-2], b.shape[-1], v.shape[-1]
        A = np.exp(A_log) if mutation == "A_positive" else -np.exp(A_log)
        out = np.zeros(v.shape)
        hT = np.zeros((len(spans), H, S, Dv))
        carry = None
        for n, (s0, e0) in enumerate(spans):
            if mutation == "no_reset_between_sequences" and cu is not None and carry is not None:
                st = carry
            elif h0 is None or mutation == "ignore_h0":
                st = np.zeros((H, S, Dv))
            else:
                st = np.array(h0[n], dtype=np.float64)
            prev = np.zeros(H)
            for t in range(s0, e0):
                i = sel(n, t)
                gt = g[i]
                if mutation == "decay_off_by_one":
                    gt, prev = prev, g[i]
                alpha = np.exp(gt[:, None] * A)
                if mutation == "decay_per_value_column":
                    alpha = alpha[:, :Dv] if Dv <= S else np.pad(alpha, ((0, 0), (0, Dv - S)), constant_values=1)
                    upd = alpha[:, None, :] * st
                else:
                    upd = alpha[:, :, None] * st
                bt, ct = b[i], c[i]
                if mutation == "swap_b_c":
                    bt, ct = ct, bt
                write = bt[:, :, None] * v[i][:, None, :]
                if mutation == "decay_after_write":
                    st = alpha[:, :, None] * (st + write)
                elif mutation == "read_before_write":
                    o = np.einsum("hs,hsd->hd", ct, st)
                    st = upd + write
                    out[i] = o
                    continue
                else:
                    st = upd + write
                out[i] = np.einsum("hs,hsd->hd", ct, st)
            hT[n] = st
            carry = st
        if D is not None:
            Dk = np.asarray(D, dtype=np.float64)
            if mutation == "skip_after_gate":
                pass
            else:
                out = out + Dk[:, None] * v
        if gate is not None:
            if mutation == "gate_ignored":
                pass
            else:
                out = out * np.asarray(gate, dtype=np.float64)[..., None]
        if D is not None and mutation == "skip_after_gate":
            out = out + np.asarray(D, dtype=np.float64)[:, None] * v
        return out, hT

    return fwd


MUTATIONS = ["A_positive", "no_reset_between_sequences", "ignore_h0", "decay_off_by_one",
             "decay_per_value_column", "swap_b_c", "decay_after_write", "read_before_write",
             "skip_after_gate", "gate_ignored"]


def test_unmutated_copy_passes():
    fwd = _mutant("none")
    for pin in ALL_PINS:
        pin(fwd, np.random.default_rng(4321))


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_mutant_is_caught(mutation):
    fwd = _mutant(mutation)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(fwd, np.random.default_rng(4321))
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the mistake {mutation!r}"
