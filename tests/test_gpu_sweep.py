"""Seeded sweep of random configurations against the FP64 oracles (forward,
diagonal-decay and backward entry points): shapes,
dtypes, chunk lengths, dense or packed batches (with empty and ragged
sequences), with or without an initial state, lengths that do and do not
trigger sequence segments.  Every case is fixed by its seed."""
import numpy as np
import pytest

import synth
import synth.diag as sd
from hip_case import TOL, compare, run_hip, run_hip_recurrent

pytestmark = pytest.mark.gpu


def _gdn_case(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    chunk = int(rng.choice([32, 64])) if dtype == "bf16" else int(rng.choice([16, 32]))
    dk, dv = int(rng.choice([32, 64, 128])), int(rng.choice([32, 64, 128]))
    H = int(rng.integers(1, 5))
    h0 = float(rng.choice([0.0, 0.2]))
    g_mean = float(rng.choice([0.0, -2.0, -4.0]))
    if rng.random() < 0.4:
        n = int(rng.integers(1, 6))
        lens = [int(x) for x in rng.integers(0, 700, size=n)]
        return synth.custom(name=f"sweep{seed}", seed=seed, H=H, dk=dk, dv=dv, dtype=dtype,
                            chunk=chunk, h0_std=h0, g_mean=g_mean, seq_lens=lens)
    B = int(rng.integers(1, 3))
    T = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(1024, 2600))]))
    return synth.custom(name=f"sweep{seed}", seed=seed, B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype,
                        chunk=chunk, h0_std=h0, g_mean=g_mean)


@pytest.mark.parametrize("seed", range(24))
def test_gdn_random_configuration(seed):
    wl = _gdn_case(seed)
    inp = synth.generate(wl)
    print(wl, flush=True)
    out, hT = run_hip(inp)
    eo, eh = compare(inp, out, hT)
    tol = TOL[wl.dtype]
    print(f"chunked: rel err out {eo:.2e} hT {eh:.2e}", flush=True)
    assert eo <= tol and eh <= tol
    if wl.tokens <= 800:
        out, hT = run_hip_recurrent(inp)
        eo, eh = compare(inp, out, hT)
        print(f"token-by-token: rel err out {eo:.2e} hT {eh:.2e}", flush=True)
        assert eo <= tol and eh <= tol


@pytest.mark.parametrize("seed", range(12))
def test_diag_random_configuration(seed):
    from test_gpu_diag import check

    rng = np.random.default_rng(2000 + seed)
    H = int(rng.integers(1, 6))
    h0 = float(rng.choice([0.0, 0.2]))
    epi = bool(rng.random() < 0.7)
    if rng.random() < 0.4:
        lens = [int(x) for x in rng.integers(0, 500, size=int(rng.integers(1, 5)))]
        wl = sd.custom(f"dsweep{seed}", seed=seed, H=H, dtype="bf16", h0_std=h0, epilogue=epi,
                       seq_lens=lens)
    else:
        T = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(600, 2100))]))
        wl = sd.custom(f"dsweep{seed}", seed=seed, B=int(rng.integers(1, 3)), T=T, H=H,
                       dtype="bf16", h0_std=h0, epilogue=epi)
    print(wl, flush=True)
    inp = sd.generate(wl)
    check(inp, "chunked")
    if wl.tokens <= 600:
        check(inp, "recurrent")


@pytest.mark.parametrize("seed", range(12))
def test_bwd_random_configuration(seed):
    """The backward entry point on random shapes, dtypes, packings, initial
    states, decays and output gradients (with and without dhT)."""
    from test_gpu_bwd import _check

    rng = np.random.default_rng(3000 + seed)
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    dk, dv = int(rng.choice([32, 64, 128])), int(rng.choice([32, 64, 128]))
    H = int(rng.integers(1, 4))
    h0 = float(rng.choice([0.0, 0.2]))
    g_mean = float(rng.choice([0.0, -2.0]))
    dh = float(rng.choice([0.0, 1.0]))
    if rng.random() < 0.4:
        lens = [int(x) for x in rng.integers(0, 300, size=int(rng.integers(1, 5)))]
        wl = synth.custom(name=f"bwd_sweep{seed}", seed=seed, H=H, dk=dk, dv=dv, dtype=dtype,
                          h0_std=h0, g_mean=g_mean, seq_lens=lens)
    else:
        wl = synth.custom(name=f"bwd_sweep{seed}", seed=seed, B=int(rng.integers(1, 3)),
                          T=int(rng.integers(1, 400)), H=H, dk=dk, dv=dv, dtype=dtype,
                          h0_std=h0, g_mean=g_mean)
    inp = synth.generate(wl)
    print(wl, flush=True)
    _check(inp, synth.output_grads(inp, 4000 + seed, dh))
