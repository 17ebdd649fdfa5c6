"""Token-by-token entry point (gdn_fwd_recurrent) vs the FP64 oracle,
element by element, through the C ABI.

Tolerances as for the chunkwise entry point: 1e-4 (float32 storage) and 2e-2
(bfloat16 storage); this form computes in fp32 throughout, so it lands well
inside both.  Index handling (packing, aliasing, determinism) is checked bit
for bit against other GPU runs.
"""
import pytest

import synth
from hip_case import TOL, compare, dev, device_inputs, run_hip_recurrent

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _check(inp, chains=None, tol=None):
    out, hT = run_hip_recurrent(inp)
    eo, eh = compare(inp, out, hT, chains)
    tol = tol if tol is not None else TOL[inp.wl.dtype]
    print(f"{inp.wl.name}: rel err out {eo:.3e} hT {eh:.3e} (tol {tol:g})", flush=True)
    assert eo <= tol and eh <= tol, (eo, eh)
    return out, hT


def test_tiny_workload():
    _check(synth.generate(synth.WORKLOADS["tiny"]))


CASES = [
    # (dtype, B, T, H, dk, dv, h0_std)
    ("f32", 2, 1, 3, 32, 32, 0.3),
    ("f32", 1, 37, 2, 64, 32, 0.3),
    ("f32", 1, 20, 2, 128, 64, 0.0),
    ("f32", 2, 9, 2, 32, 128, 0.5),
    ("f32", 1, 64, 2, 128, 128, 0.3),
    ("bf16", 4, 1, 4, 128, 128, 0.02),
    ("bf16", 2, 16, 3, 128, 128, 0.3),
    ("bf16", 3, 5, 2, 32, 32, 0.3),
    ("bf16", 2, 7, 2, 64, 64, 0.0),
    ("bf16", 1, 33, 3, 32, 128, 0.2),
    ("bf16", 1, 12, 3, 128, 32, 0.2),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_shapes(case):
    dtype, B, T, H, dk, dv, h0 = case
    wl = synth.custom(name="rec", seed=200 + CASES.index(case), B=B, T=T, H=H, dk=dk, dv=dv,
                      dtype=dtype, chunk=64 if dtype == "bf16" else 16, h0_std=h0)
    _check(synth.generate(wl))


def test_decode_batch_sampled_chains():
    """A decoding step at batch scale (one token per sequence, d=128, nonzero
    state), sampled chains against the oracle."""
    wl = synth.custom(name="decode", seed=5, B=128, T=1, H=16, dk=128, dv=128, dtype="bf16",
                      chunk=64, h0_std=0.02)
    inp = synth.generate(wl)
    _check(inp, chains=[0, 1, 17, 500, 1023, 1500, 2047])


def test_slow_decay_long_sequence_f32():
    wl = synth.custom(name="rec-long", seed=210, B=1, T=300, H=2, dk=64, dv=64, dtype="f32",
                      chunk=16, h0_std=0.5, g_mean=-3.0)
    _check(synth.generate(wl))


def test_packed_with_empty_sequences():
    wl = synth.custom(name="rec-pk", seed=211, H=2, dk=128, dv=128, dtype="bf16", chunk=64,
                      seq_lens=[5, 0, 1, 17, 0, 3])
    _check(synth.generate(wl))


def test_packed_equals_per_sequence_bitwise():
    lens = [9, 0, 4, 1, 13]
    wl = synth.custom(name="rec-pk2", seed=212, H=2, dk=64, dv=128, dtype="bf16", chunk=64,
                      seq_lens=lens)
    inp = synth.generate(wl)
    d = device_inputs(inp)
    h0 = torch.randn(len(lens), 2, 64, 128, device="cuda") * 0.1
    d["h0"] = h0
    out, hT = run_hip_recurrent(inp, d=d)
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        s, e = int(cu[n]), int(cu[n + 1])
        one = dict(q=d["q"][s:e][None].contiguous(), k=d["k"][s:e][None].contiguous(),
                   v=d["v"][s:e][None].contiguous(), g=d["g"][s:e][None].contiguous(),
                   beta=d["beta"][s:e][None].contiguous(), h0=h0[n:n + 1].contiguous(),
                   cu_seqlens=None)
        o1, h1 = run_hip_recurrent(inp, d=one)
        assert torch.equal(_bits(out[s:e]), _bits(o1[0])), f"sequence {n} out"
        assert torch.equal(_bits(hT[n]), _bits(h1[0])), f"sequence {n} hT"


def test_steps_compose_bitwise():
    """Running tokens [0, t) and then [t, T) from the first call's state is
    the same computation as one call over [0, T)."""
    wl = synth.custom(name="rec-split", seed=213, B=2, T=12, H=2, dk=128, dv=128, dtype="bf16",
                      chunk=64, h0_std=0.3)
    inp = synth.generate(wl)
    d = device_inputs(inp)
    out, hT = run_hip_recurrent(inp, d=d)
    part = lambda lo, hi, h0: dict(
        q=d["q"][:, lo:hi].contiguous(), k=d["k"][:, lo:hi].contiguous(),
        v=d["v"][:, lo:hi].contiguous(), g=d["g"][:, lo:hi].contiguous(),
        beta=d["beta"][:, lo:hi].contiguous(), h0=h0, cu_seqlens=None)
    oa, ha = run_hip_recurrent(inp, d=part(0, 5, d["h0"]))
    ob, hb = run_hip_recurrent(inp, d=part(5, 12, ha))
    assert torch.equal(_bits(torch.cat([oa, ob], dim=1)), _bits(out))
    assert torch.equal(_bits(hb), _bits(hT))


def test_agrees_with_chunkwise_form():
    from hip_case import run_hip

    wl = synth.custom(name="rec-vs-chunk", seed=214, B=1, T=70, H=2, dk=128, dv=128,
                      dtype="f32", chunk=16, h0_std=0.3)
    inp = synth.generate(wl)
    d = device_inputs(inp)
    o1, h1 = run_hip_recurrent(inp, d=d)
    o2, h2 = run_hip(inp, d=d)
    scale_o = float(o2.abs().max())
    scale_h = float(h2.abs().max())
    assert float((o1 - o2).abs().max()) <= 1e-4 * scale_o
    assert float((h1 - h2).abs().max()) <= 1e-4 * scale_h


def test_deterministic_and_hT_may_alias_h0():
    inp = synth.generate(synth.custom(name="rec-alias", seed=215, B=2, T=6, H=2, dk=64, dv=64,
                                      dtype="bf16", chunk=64, h0_std=0.5))
    d = device_inputs(inp)
    o1, h1 = run_hip_recurrent(inp, d=d)
    o2, h2 = run_hip_recurrent(inp, d=d)
    assert torch.equal(_bits(o1), _bits(o2)) and torch.equal(_bits(h1), _bits(h2))
    state = d["h0"].clone()
    d["h0"] = state
    o3, h3 = run_hip_recurrent(inp, d=d, hT=state)
    assert h3.data_ptr() == state.data_ptr()
    assert torch.equal(_bits(o1), _bits(o3)) and torch.equal(_bits(h1), _bits(state))


def test_empty_inputs():
    inp = synth.generate(synth.custom(name="rec-empty", seed=216, B=2, T=0, H=2, dk=32, dv=32,
                                      dtype="bf16", chunk=64, h0_std=0.5))
    out, hT = run_hip_recurrent(inp)
    assert out.numel() == 0
    assert torch.equal(hT, dev(inp.h0))
