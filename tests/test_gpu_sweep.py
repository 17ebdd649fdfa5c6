"""Seeded sweep of random configurations against the FP64 oracles (forward,
diagonal-decay and backward entry points, and the training pair against the
plain forward and backward): shapes,
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


@pytest.mark.parametrize("seed", range(8))
def test_train_random_configuration(seed):
    """The training pair on random full-width cases (bf16, dk = dv = 128):
    gdn_fwd_train's out and hT equal gdn_fwd's bit for bit, and gdn_bwd_saved
    from its records equals gdn_bwd bit for bit, dense (lengths that are and
    are not cut into segments) and packed (with empty and ragged sequences);
    small cases also against the FP64 oracle."""
    import torch

    import gated_deltanet_recurrence_delta_amd as gdn
    from hip_case import dev, host_f64
    from test_gpu_bwd import NAMES, _oracle, _rel

    rng = np.random.default_rng(5000 + seed)
    H = int(rng.integers(1, 5))
    h0 = float(rng.choice([0.0, 0.2]))
    g_mean = float(rng.choice([0.0, -2.0, -4.0]))
    dh = float(rng.choice([0.0, 1.0]))
    if rng.random() < 0.4:
        lens = [int(x) for x in rng.integers(0, 1400, size=int(rng.integers(1, 5)))]
        wl = synth.custom(name=f"train_sweep{seed}", seed=seed, H=H, dk=128, dv=128, dtype="bf16",
                          h0_std=h0, g_mean=g_mean, seq_lens=lens)
    else:
        T = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(1024, 2200))]))
        wl = synth.custom(name=f"train_sweep{seed}", seed=seed, B=int(rng.integers(1, 3)), T=T, H=H,
                          dk=128, dv=128, dtype="bf16", h0_std=h0, g_mean=g_mean)
    inp = synth.generate(wl)
    og = synth.output_grads(inp, 6000 + seed, dh)
    print(wl, flush=True)
    d = {n: dev(getattr(inp, n)) for n in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")}
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"])
    out1, hT1 = gdn.fwd(*args)
    out2, hT2, ws = gdn.fwd_train(*args)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(hT1.view(torch.int32), hT2.view(torch.int32))
    kw = dict(h0=d["h0"], cu_seqlens=d["cu_seqlens"], dhT=dev(og.dhT))
    g1 = gdn.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dev(og.dout), **kw)
    g2 = gdn.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dev(og.dout), workspace=ws, saved=True, **kw)
    torch.cuda.synchronize()
    for n in NAMES:
        if g1[n] is not None:
            assert torch.equal(g1[n], g2[n]), n
    if wl.tokens * H <= 3000:
        ref = _oracle(inp, og)
        for n in NAMES:
            e = _rel(host_f64(g2[n]), ref[n])
            assert e <= TOL["bf16"], (n, e)
