"""The chunk-map scan entry point (gdn_fwd_scan) against the FP64 oracle,
through the C ABI.

A sequence of more than 16 chunks runs as segments whose exact entry states
come from the segments' affine maps (M_end = P M_start + Q) and a short
scan.  Checked here: the maps and entry states the call leaves in its
workspace against ``oracle/scan.py`` and the sequential oracle; outputs and
hT on every chain of long_context with no decay and with its own slow
decay; ragged tails, packed batches (bitwise equal to each sequence alone),
aliasing, workspace reuse and the shapes that fall back to the uncut path.
Tolerance: the bf16 one, 2e-2 infinity-norm relative, per tensor and per
chain.
"""
import numpy as np
import pytest

import oracle
import synth
from hip_case import TOL, compare_all, device_inputs, host_f64, run_hip, run_hip_scan
from oracle import scan

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DK = DV = 128
SEG_MAX = 16


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _seg_len(nch):
    """Segment length in chunks of a sequence of nch chunks (ceil(nch / 16)
    equal segments)."""
    n0 = -(-nch // SEG_MAX)
    return -(-nch // n0)


def _check(inp, **kw):
    out, hT = run_hip_scan(inp, **kw)
    r = compare_all(inp, out, hT)
    tol = TOL[inp.wl.dtype]
    print(f"{inp.wl.name} (scan): rel err out {r['out']:.3e} hT {r['hT']:.3e}; worst chain "
          f"{r['worst_chain']} out {r['chain_out']:.3e} hT {r['chain_hT']:.3e} (tol {tol:g})",
          flush=True)
    assert max(r["out"], r["hT"], r["chain_out"], r["chain_hT"]) <= tol, r
    return out, hT


def _workspace(inp):
    import gated_deltanet_recurrence_delta_amd as gdn

    wl = inp.wl
    packed = inp.cu_seqlens is not None
    B = len(inp.cu_seqlens) - 1 if packed else wl.B
    T = int(inp.cu_seqlens[-1]) if packed else wl.T
    need = gdn.gdn_fwd_scan_workspace_size(B, T, wl.H, wl.dk, wl.dv, packed, gdn.GDN_BF16, wl.chunk)
    assert need > 0
    return torch.zeros(need, dtype=torch.uint8, device="cuda")


def _rel(x, ref):
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-300))


@pytest.mark.parametrize("decay", ["none", "slow"])
def test_maps_and_entry_states_against_oracle(decay):
    """One dense 40-chunk sequence per batch entry, with h0: cut into
    segments of 14, 14 and 12 chunks.  The workspace then holds Q_0, (P_1,
    Q_1) and the entry states S_0..S_2; each is compared with the FP64
    chunk maps of oracle/scan.py and with the sequential oracle's state at
    the segment boundary."""
    wl = synth.custom(name=f"maps_{decay}", seed=61, B=2, T=40 * 64, H=2, dk=DK, dv=DV,
                      dtype="bf16", chunk=64, h0_std=0.5, g_mean=-4.0, no_decay=decay == "none")
    inp = synth.generate(wl)
    ws = _workspace(inp)
    _check(inp, workspace=ws)
    nch, L = 40, _seg_len(40)
    assert L == 14
    nseg = -(-nch // L)
    W = ws.view(torch.float32).view(wl.B * nseg, wl.H, 3, DK, DV).cpu().numpy().astype(np.float64)
    f = {n: inp.as_f64(n) for n in ("q", "k", "v", "g", "beta", "h0")}
    for b in range(wl.B):
        for h in range(wl.H):
            k, v, g, beta = f["k"][b, :, h], f["v"][b, :, h], f["g"][b, :, h], f["beta"][b, :, h]
            maps = scan.segment_maps(k, v, g, beta, 64, L)
            # entry states from the sequential oracle on each prefix
            for s in range(nseg):
                t = s * L * 64
                if t == 0:
                    ref = f["h0"][b, h]
                else:
                    sel = lambda x: x[b:b + 1, :t]
                    _, hT = oracle.fwd_seq(sel(f["q"]), sel(f["k"]), sel(f["v"]), sel(f["g"]),
                                           sel(f["beta"]), f["h0"][b:b + 1])
                    ref = hT[0, h]
                got = W[b * nseg + s, h, 2]
                assert _rel(got, ref) <= 2e-2, (b, h, s, "S", _rel(got, ref))
            # Q_0 starts from h0: it is the second segment's entry state
            P0, Q0 = maps[0]
            assert _rel(W[b * nseg, h, 1], P0 @ f["h0"][b, h] + Q0) <= 2e-2, (b, h, "Q0")
            for s in range(1, nseg - 1):
                P, Q = maps[s]
                assert _rel(W[b * nseg + s, h, 0], P) <= 2e-2, (b, h, s, "P", _rel(W[b * nseg + s, h, 0], P))
                assert _rel(W[b * nseg + s, h, 1], Q) <= 2e-2, (b, h, s, "Q", _rel(W[b * nseg + s, h, 1], Q))


@pytest.mark.parametrize("name", ["long_context_nodecay", "long_context"])
def test_long_context_every_chain(name):
    """B=1 H=16 T=32,768 d=128: 512 chunks in 16 segments per chain on 256
    CUs, every chain against the oracle -- with no decay at all (where the
    halo segments of gdn_fwd reach back to the sequence start) and with
    long_context's slow decay."""
    _check(synth.generate(synth.WORKLOADS[name]))


def test_no_decay_scan_equals_uncut_within_rounding():
    """The scan and the uncut chunk recurrence agree on every element
    within the bf16 tolerance (both carry the state in fp32)."""
    inp = synth.generate(synth.custom(name="nd_uncut", seed=62, B=1, T=3000, H=4, dk=DK, dv=DV,
                                      dtype="bf16", chunk=64, h0_std=0.3, no_decay=True))
    d = device_inputs(inp)
    o1, h1 = run_hip_scan(inp, d=d)
    o2, h2 = run_hip(inp, d=d, segments=False)
    assert oracle.rel_err(host_f64(o1), host_f64(o2)) <= 2e-2
    assert oracle.rel_err(host_f64(h1), host_f64(h2)) <= 2e-2


@pytest.mark.parametrize("T", [1025, 2000, 16 * 64 + 63, 4096 + 1])
def test_ragged_lengths(T):
    """Lengths just past the cut (17 chunks, the last one token), ragged
    tails, with h0 and no decay."""
    _check(synth.generate(synth.custom(name=f"rag{T}", seed=63, B=2, T=T, H=3, dk=DK, dv=DV,
                                       dtype="bf16", chunk=64, h0_std=0.4, no_decay=True)))


def test_packed_every_chain_and_bitwise_alone():
    """A packed batch with empty, short, uncut and cut sequences (up to 5
    segments), no decay: every chain against the oracle, and every
    sequence's slice equal to that sequence run alone bit for bit."""
    lens = [3000, 0, 64, 1500, 1025, 1, 5000, 1024, 700]
    inp = synth.generate(synth.custom(name="scan_pk", seed=64, H=3, dk=DK, dv=DV, dtype="bf16",
                                      chunk=64, no_decay=True, seq_lens=lens))
    d = device_inputs(inp)
    nseq = len(lens)
    d["h0"] = torch.randn(nseq, 3, DK, DV, device="cuda",
                          generator=torch.Generator(device="cuda").manual_seed(5)) * 0.3
    inp.h0 = d["h0"].cpu().numpy()
    out, hT = _check(inp, d=d)
    cu = inp.cu_seqlens
    for n in range(nseq):
        s, e = int(cu[n]), int(cu[n + 1])
        one = {m: d[m][s:e][None].contiguous() for m in ("q", "k", "v", "g", "beta")}
        one.update(h0=d["h0"][n:n + 1].contiguous(), cu_seqlens=None)
        o1, h1 = run_hip_scan(inp, d=one)
        assert torch.equal(_bits(out[s:e]), _bits(o1[0])), f"sequence {n} ({e - s} tokens) out"
        assert torch.equal(_bits(hT[n]), _bits(h1[0])), f"sequence {n} ({e - s} tokens) hT"


def test_varlen_workload_every_chain():
    """The varlen workload (32 sequences of 256..4,096 tokens) through the
    scan entry point."""
    _check(synth.generate(synth.WORKLOADS["varlen"]))


def test_hT_may_alias_h0():
    import gated_deltanet_recurrence_delta_amd as gdn

    inp = synth.generate(synth.custom(name="scan_alias", seed=65, B=2, T=2500, H=2, dk=DK, dv=DV,
                                      dtype="bf16", chunk=64, h0_std=0.5, no_decay=True))
    d = device_inputs(inp)
    o_ref, h_ref = run_hip_scan(inp, d=d)
    state = d["h0"].clone()
    out, hT = gdn.fwd_scan(d["q"], d["k"], d["v"], d["g"], d["beta"], state, None, chunk=64, hT=state)
    torch.cuda.synchronize()
    assert hT.data_ptr() == state.data_ptr()
    assert torch.equal(_bits(out), _bits(o_ref)) and torch.equal(_bits(hT), _bits(h_ref))


def test_workspace_reuse_across_calls():
    """Two calls in a row on one workspace, the second on other inputs and
    a shorter sequence: each equals the same call on a fresh workspace."""
    a = synth.generate(synth.custom(name="ws_a", seed=66, B=1, T=4000, H=2, dk=DK, dv=DV,
                                    dtype="bf16", chunk=64, h0_std=0.3, no_decay=True))
    b = synth.generate(synth.custom(name="ws_b", seed=67, B=1, T=2100, H=2, dk=DK, dv=DV,
                                    dtype="bf16", chunk=64, g_mean=-4.0))
    ws = _workspace(a)
    ra = run_hip_scan(a, workspace=ws)
    rb = run_hip_scan(b, workspace=ws)
    fa = run_hip_scan(a, workspace=_workspace(a))
    fb = run_hip_scan(b, workspace=_workspace(b))
    for x, y in zip(ra + rb, fa + fb):
        assert torch.equal(_bits(x), _bits(y))


def test_other_shapes_run_uncut():
    """d = 32 has no scan: the call equals gdn_fwd without segments."""
    inp = synth.generate(synth.custom(name="scan_d32", seed=68, B=2, T=3000, H=4, dk=32, dv=32,
                                      dtype="bf16", chunk=64, no_decay=True))
    d = device_inputs(inp)
    o1, h1 = run_hip_scan(inp, d=d)
    o2, h2 = run_hip(inp, d=d, segments=False)
    assert torch.equal(_bits(o1), _bits(o2)) and torch.equal(_bits(h1), _bits(h2))
    _check(inp, d=d)


def test_short_sequences_need_no_workspace():
    """At most 16 chunks per sequence: nothing is cut, the workspace size is
    0 and the call equals gdn_fwd's."""
    inp = synth.generate(synth.custom(name="scan_short", seed=69, B=3, T=1024, H=2, dk=DK, dv=DV,
                                      dtype="bf16", chunk=64, h0_std=0.2, no_decay=True))
    d = device_inputs(inp)
    o1, h1 = run_hip_scan(inp, d=d)
    o2, h2 = run_hip(inp, d=d)
    assert torch.equal(_bits(o1), _bits(o2)) and torch.equal(_bits(h1), _bits(h2))
