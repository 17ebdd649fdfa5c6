"""Each plausible mistake planted in a copy of the sequential rule must break
at least one pin: this is what makes the pins a check of the oracle rather
than a restatement of it.  Mistakes are planted on the CPU, in this file's
own copies; the oracle itself is untouched."""
import numpy as np
import pytest

from pins import ALL_PINS


def _make(mutation):
    """Sequential rule in the M = S^T orientation with one planted mistake."""

    def fwd(q, k, v, g, beta, h0=None, cu=None):
        q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
        if cu is not None:
            T, H, dk = q.shape
            B = len(cu) - 1
            spans = [(int(cu[b]), int(cu[b + 1])) for b in range(B)]
            sel = lambda b, h, t: (t, h)
        else:
            B, T, H, dk = q.shape
            spans = [(0, T)] * B
            sel = lambda b, h, t: (b, t, h)
        dv = v.shape[-1]
        out = np.zeros(v.shape)
        hT = np.zeros((B, H, dk, dv))
        carry = {}
        for b in range(B):
            for h in range(H):
                if mutation == "no_reset_between_sequences" and cu is not None and h in carry:
                    M = carry[h].copy()
                elif h0 is None or mutation == "ignore_h0":
                    M = np.zeros((dk, dv))
                else:
                    M = np.array(h0[b, h], dtype=np.float64)
                s, e = spans[b]
                prev_g = 0.0
                for t in range(s, e):
                    i = sel(b, h, t)
                    kt, qt, vt = k[i], q[i], v[i]
                    if mutation == "swap_q_k":
                        kt, qt = qt, kt
                    gt = g[i]
                    if mutation == "decay_off_by_one":
                        gt, prev_g = prev_g, g[i]
                    a = np.exp(-gt) if mutation == "exp_minus_g" else np.exp(gt)
                    bt = beta[i]
                    M_prev = M
                    p = M.T @ kt
                    if mutation == "no_erase":
                        M = a * M + bt * np.outer(kt, vt)
                    elif mutation == "erase_sign":
                        M = a * M + bt * np.outer(kt, vt + a * p)
                    elif mutation == "prediction_without_decay":
                        M = a * M + bt * np.outer(kt, vt - p)
                    elif mutation == "decay_after_write":
                        M = a * (M + bt * np.outer(kt, vt - p))
                    elif mutation == "beta_on_value_only":
                        M = a * M + np.outer(kt, bt * vt - a * p)
                    elif mutation == "erase_uses_query":
                        M = a * M + bt * np.outer(kt, vt - a * (M.T @ qt))
                    else:
                        M = a * M + bt * np.outer(kt, vt - a * p)
                    if mutation == "read_before_write":
                        out[i] = M_prev.T @ qt
                    elif mutation == "transposed_read":
                        out[i] = M @ qt[: M.shape[1]] if M.shape[0] == M.shape[1] else (M.T @ qt)[::-1]
                    else:
                        out[i] = M.T @ qt
                hT[b, h] = M.T if (mutation == "transposed_state_out" and dk == dv) else (
                    M.T.reshape(dk, dv) if mutation == "transposed_state_out" else M)
                carry[h] = M
        return out, hT

    return fwd


MUTATIONS = ["no_erase", "erase_sign", "prediction_without_decay", "decay_after_write",
             "beta_on_value_only", "erase_uses_query", "read_before_write",
             "transposed_read", "swap_q_k", "decay_off_by_one", "exp_minus_g",
             "ignore_h0", "no_reset_between_sequences", "transposed_state_out"]


def _broken_pins(fwd):
    broken = []
    for pin in ALL_PINS:
        try:
            pin(fwd, np.random.default_rng(1234))
        except (AssertionError, ValueError, IndexError):
            broken.append(pin.__name__)
    return broken


def test_unmutated_copy_passes_all_pins():
    assert _broken_pins(_make("none")) == []


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_mutant_breaks_a_pin(mutation):
    assert _broken_pins(_make(mutation)), f"no pin detects mutation {mutation!r}"
