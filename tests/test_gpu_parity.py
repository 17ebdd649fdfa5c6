"""HIP path vs the FP64 oracle, element by element, through the C ABI.

Tolerances (infinity-norm relative error per output tensor, out and hT
separately): 1e-4 for float32 storage, 2e-2 for bfloat16 storage with fp32
accumulation.  Index handling (packing, chunk boundaries, causality,
aliasing, determinism) is checked bit for bit against other GPU runs.
"""
import dataclasses

import numpy as np
import pytest

import synth
from hip_case import TOL, compare, compare_all, dev, device_inputs, host_f64, run_hip

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _check(inp, chunk=None, **kw):
    """Every chain against the oracle: the whole-tensor error and each
    chain's error on its own scale must be within the tolerance."""
    out, hT = run_hip(inp, chunk=chunk, **kw)
    r = compare_all(inp, out, hT)
    tol = TOL[inp.wl.dtype]
    print(f"{inp.wl.name}: rel err out {r['out']:.3e} hT {r['hT']:.3e}; worst chain "
          f"{r['worst_chain']} out {r['chain_out']:.3e} hT {r['chain_hT']:.3e} (tol {tol:g})",
          flush=True)
    assert max(r["out"], r["hT"], r["chain_out"], r["chain_hT"]) <= tol, r
    return out, hT


# ------------------------------------------------------------ full oracle --

def test_tiny_workload():
    _check(synth.generate(synth.WORKLOADS["tiny"]))


SMALL = [
    # (dtype, B, T, H, dk, dv, chunk, h0_std)
    ("f32", 2, 200, 3, 32, 32, 16, 0.3),
    ("f32", 1, 77, 2, 64, 32, 32, 0.3),
    ("f32", 1, 90, 2, 128, 64, 32, 0.0),
    ("f32", 1, 130, 2, 32, 128, 32, 0.5),
    ("bf16", 2, 200, 3, 128, 128, 64, 0.3),
    ("bf16", 1, 333, 2, 128, 128, 32, 0.0),
    ("bf16", 3, 150, 2, 32, 32, 64, 0.3),
    ("bf16", 2, 97, 2, 64, 64, 64, 0.3),
    ("bf16", 1, 129, 3, 32, 128, 64, 0.2),
    ("bf16", 1, 129, 3, 128, 32, 32, 0.2),
    ("bf16", 1, 10, 4, 128, 128, 64, 0.5),
    ("bf16", 1, 1, 2, 128, 128, 64, 0.5),
    ("f32", 1, 1, 2, 32, 32, 16, 0.5),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_small_shapes(case):
    dtype, B, T, H, dk, dv, chunk, h0 = case
    wl = synth.custom(name="small", seed=100 + SMALL.index(case), B=B, T=T, H=H, dk=dk, dv=dv,
                      dtype=dtype, chunk=chunk, h0_std=h0)
    _check(synth.generate(wl))


def test_slow_decay_keeps_h0_visible():
    """Slow decay so that h0 still shows in hT after many chunks."""
    wl = synth.custom(name="slow", seed=21, B=2, T=300, H=2, dk=128, dv=128, dtype="bf16",
                      chunk=64, h0_std=1.0, g_mean=-4.0)
    _check(synth.generate(wl))


def test_many_workgroups():
    """More work items than compute units: several dispatch rounds."""
    wl = synth.custom(name="wide", seed=22, B=6, T=70, H=16, dk=128, dv=128, dtype="bf16",
                      chunk=64, h0_std=0.1)
    _check(synth.generate(wl))


@pytest.mark.parametrize("dtype,chunk", [("f32", 16), ("f32", 32), ("bf16", 32), ("bf16", 64)])
def test_chunk_lengths_agree(dtype, chunk):
    wl = synth.custom(name="chunks", seed=23, B=1, T=250, H=2, dk=32, dv=32, dtype=dtype,
                      chunk=chunk, h0_std=0.2)
    _check(synth.generate(wl))


def test_packed_small():
    wl = synth.custom(name="packed", seed=24, H=3, dk=128, dv=128, dtype="bf16", chunk=64,
                      seq_lens=[65, 0, 1, 64, 200, 3, 0])
    _check(synth.generate(wl))


def test_packed_f32():
    wl = synth.custom(name="packed32", seed=25, H=2, dk=32, dv=32, dtype="f32", chunk=16,
                      h0_std=0.4, seq_lens=[17, 0, 33, 1, 16])
    _check(synth.generate(wl))


# ------------------------------------------------------- full-size workloads --

@pytest.mark.parametrize("name", ["small_state", "wide_head", "varlen", "long_context"])
def test_full_workload_every_chain(name):
    """Full size, the benchmark's launch: every chain against the oracle."""
    _check(synth.generate(synth.WORKLOADS[name]))


@pytest.mark.parametrize("name", ["wide_head", "long_context"])
def test_full_workload_uncut(name):
    """The same workloads with every chain run from its start."""
    _check(synth.generate(synth.WORKLOADS[name]), segments=False)


# ----------------------------------------------------------- bit-exactness --

def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_packed_equals_per_sequence_bitwise():
    lens = [100, 0, 64, 1, 129, 63]
    wl = synth.custom(name="pk", seed=31, H=2, dk=128, dv=128, dtype="bf16", chunk=64,
                      seq_lens=lens)
    inp = synth.generate(wl)
    d = device_inputs(inp)
    h0 = torch.randn(len(lens), 2, 128, 128, device="cuda") * 0.1
    d["h0"] = h0
    out, hT = run_hip(inp, d=d)
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        s, e = int(cu[n]), int(cu[n + 1])
        one = dict(q=d["q"][s:e][None].contiguous(), k=d["k"][s:e][None].contiguous(),
                   v=d["v"][s:e][None].contiguous(), g=d["g"][s:e][None].contiguous(),
                   beta=d["beta"][s:e][None].contiguous(), h0=h0[n:n + 1].contiguous(),
                   cu_seqlens=None)
        o1, h1 = run_hip(inp, d=one)
        assert torch.equal(_bits(out[s:e]), _bits(o1[0])), f"sequence {n} out"
        assert torch.equal(_bits(hT[n]), _bits(h1[0])), f"sequence {n} hT"


def test_length_ordered_dispatch_bitwise():
    """A packed batch (d = 64, the per-tile kernel) large enough for the
    kernel to hand out the longest sequences first (equal lengths and empty sequences included): every
    sequence is still bitwise its own single-sequence run, and within
    tolerance of the oracle."""
    lens = [70, 0, 130, 70, 1, 200, 0, 64]
    wl = synth.custom(name="lpt", seed=39, H=4, dk=64, dv=64, dtype="bf16", chunk=64,
                      seq_lens=lens)
    inp = synth.generate(wl)
    d = device_inputs(inp)
    h0 = torch.randn(len(lens), 4, 64, 64, device="cuda") * 0.1
    d["h0"] = h0
    out, hT = run_hip(inp, d=d)
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        s, e = int(cu[n]), int(cu[n + 1])
        one = dict(q=d["q"][s:e][None].contiguous(), k=d["k"][s:e][None].contiguous(),
                   v=d["v"][s:e][None].contiguous(), g=d["g"][s:e][None].contiguous(),
                   beta=d["beta"][s:e][None].contiguous(), h0=h0[n:n + 1].contiguous(),
                   cu_seqlens=None)
        o1, h1 = run_hip(inp, d=one)
        assert torch.equal(_bits(out[s:e]), _bits(o1[0])), f"sequence {n} out"
        assert torch.equal(_bits(hT[n]), _bits(h1[0])), f"sequence {n} hT"
    import dataclasses

    eo, eh = compare(dataclasses.replace(inp, h0=h0.cpu().numpy()), out, hT)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (eo, eh)


def _alone(d, s, e, h0):
    """Sequence [s, e) of a packed batch's device inputs as a dense B=1 call."""
    one = {n: d[n][s:e][None].contiguous() for n in ("q", "k", "v", "g", "beta")}
    one.update(h0=h0, cu_seqlens=None)
    return one


@pytest.mark.parametrize("segments,with_h0", [(True, False), (True, True), (False, False)])
def test_varlen_workload_packed_equals_per_sequence_bitwise(segments, with_h0):
    """The varlen workload at its real lengths (32 sequences of 256..4,096
    tokens, H=16, d=128): every sequence's slice of the packed run equals
    that sequence run alone bit for bit -- with the default cut into
    segments (which depends on the sequence alone) and without it."""
    inp = synth.generate(synth.WORKLOADS["varlen"])
    d = device_inputs(inp)
    nseq = len(inp.cu_seqlens) - 1
    wl = inp.wl
    h0 = None
    if with_h0:
        h0 = torch.randn(nseq, wl.H, wl.dk, wl.dv, device="cuda", generator=torch.Generator(
            device="cuda").manual_seed(7)) * 0.02
    d["h0"] = h0
    out, hT = run_hip(inp, d=d, segments=segments)
    cu = inp.cu_seqlens
    for n in range(nseq):
        s, e = int(cu[n]), int(cu[n + 1])
        o1, h1 = run_hip(inp, d=_alone(d, s, e, None if h0 is None else h0[n:n + 1].contiguous()),
                         segments=segments)
        assert torch.equal(_bits(out[s:e]), _bits(o1[0])), f"sequence {n} ({e - s} tokens) out"
        assert torch.equal(_bits(hT[n]), _bits(h1[0])), f"sequence {n} ({e - s} tokens) hT"


def test_capped_segments_packed_equals_per_sequence_bitwise():
    """With H = 128 heads a sequence is cut into at most CUs / 128 segments
    (two on 256 CUs): the 40-chunk sequence runs as two 20-chunk segments,
    not three of 14.  Every chain matches the oracle, and each sequence's
    slice of the packed run equals the sequence run alone bit for bit."""
    inp = synth.generate(synth.custom(name="cap_packed", seed=47, H=128, dk=128, dv=128, dtype="bf16",
                                      chunk=64, h0_std=0.2, g_mean=-2.0, seq_lens=[2560, 500, 1, 1100]))
    out, hT = _check(inp)
    d = device_inputs(inp)
    cu = inp.cu_seqlens
    for n in range(len(cu) - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        o1, h1 = run_hip(inp, d=_alone(d, s, e, d["h0"][n:n + 1].contiguous()))
        assert torch.equal(_bits(out[s:e]), _bits(o1[0])), f"sequence {n} out"
        assert torch.equal(_bits(hT[n]), _bits(h1[0])), f"sequence {n} hT"


def test_causality_bitwise():
    wl = synth.custom(name="causal", seed=32, B=1, T=256, H=2, dk=128, dv=128, dtype="bf16",
                      chunk=64, h0_std=0.2)
    inp = synth.generate(wl)
    d = device_inputs(inp)
    out, _ = run_hip(inp, d=d)
    t = 100
    d2 = {k: (v.clone() if v is not None else None) for k, v in d.items()}
    for name in ("q", "k", "v"):
        d2[name][:, t + 1:] = torch.randn_like(d2[name][:, t + 1:].float()).to(d2[name].dtype)
    d2["g"][:, t + 1:] = -torch.rand_like(d2["g"][:, t + 1:])
    d2["beta"][:, t + 1:] = torch.rand_like(d2["beta"][:, t + 1:])
    out2, _ = run_hip(inp, d=d2)
    assert torch.equal(_bits(out[:, : t + 1]), _bits(out2[:, : t + 1]))
    assert not torch.equal(out[:, t + 1:], out2[:, t + 1:])


@pytest.mark.parametrize("split", [64, 128, 192])
def test_split_at_chunk_boundary_bitwise(split):
    wl = synth.custom(name="split", seed=33, B=2, T=256, H=2, dk=128, dv=128, dtype="bf16",
                      chunk=64, h0_std=0.3)
    inp = synth.generate(wl)
    d = device_inputs(inp)
    out, hT = run_hip(inp, d=d)
    part = lambda lo, hi, h0: dict(
        q=d["q"][:, lo:hi].contiguous(), k=d["k"][:, lo:hi].contiguous(),
        v=d["v"][:, lo:hi].contiguous(), g=d["g"][:, lo:hi].contiguous(),
        beta=d["beta"][:, lo:hi].contiguous(), h0=h0, cu_seqlens=None)
    oa, ha = run_hip(inp, d=part(0, split, d["h0"]))
    ob, hb = run_hip(inp, d=part(split, 256, ha))
    assert torch.equal(_bits(torch.cat([oa, ob], dim=1)), _bits(out))
    assert torch.equal(_bits(hb), _bits(hT))


def test_split_long_sequence_uncut_bitwise():
    """Without segments, a 2,048-token run split at token 1,024 (the second
    call starting from the first call's hT) equals the whole run bit for bit."""
    wl = synth.custom(name="split_long", seed=45, B=2, T=2048, H=2, dk=128, dv=128,
                      dtype="bf16", chunk=64, h0_std=0.3, g_mean=-3.0)
    inp = synth.generate(wl)
    d = device_inputs(inp)
    out, hT = run_hip(inp, d=d, segments=False)
    part = lambda lo, hi, h0: dict(
        q=d["q"][:, lo:hi].contiguous(), k=d["k"][:, lo:hi].contiguous(),
        v=d["v"][:, lo:hi].contiguous(), g=d["g"][:, lo:hi].contiguous(),
        beta=d["beta"][:, lo:hi].contiguous(), h0=h0, cu_seqlens=None)
    oa, ha = run_hip(inp, d=part(0, 1024, d["h0"]), segments=False)
    ob, hb = run_hip(inp, d=part(1024, 2048, ha), segments=False)
    assert torch.equal(_bits(torch.cat([oa, ob], dim=1)), _bits(out))
    assert torch.equal(_bits(hb), _bits(hT))


def test_guard_regions_untouched():
    """Outputs placed between guard regions filled with a sentinel: packed
    ragged sequences (empty, one-token and partial-chunk ones) and a dense
    segmented run write nothing outside out and hT."""
    import gated_deltanet_recurrence_delta_amd as gdn

    G = 4096  # guard elements on each side
    cases = [synth.custom(name="guard_pk", seed=46, H=3, dk=128, dv=128, dtype="bf16", chunk=64,
                          seq_lens=[65, 0, 1, 64, 1100, 3, 0, 127]),
             synth.custom(name="guard_dense", seed=47, B=2, T=1500, H=2, dk=128, dv=128,
                          dtype="bf16", chunk=64, h0_std=0.2),
             synth.custom(name="guard_small", seed=48, H=2, dk=32, dv=32, dtype="bf16", chunk=64,
                          seq_lens=[70, 0, 1, 130])]
    for wl in cases:
        inp = synth.generate(wl)
        d = device_inputs(inp)
        nb = len(inp.cu_seqlens) - 1 if inp.cu_seqlens is not None else wl.B
        o_buf = torch.full((G + d["v"].numel() + G,), -7.25, dtype=d["v"].dtype, device="cuda")
        h_buf = torch.full((G + nb * wl.H * wl.dk * wl.dv + G,), -7.25, device="cuda")
        out = o_buf[G:G + d["v"].numel()].view(d["v"].shape)
        hT = h_buf[G:G + nb * wl.H * wl.dk * wl.dv].view(nb, wl.H, wl.dk, wl.dv)
        gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                chunk=wl.chunk, out=out, hT=hT)
        torch.cuda.synchronize()
        for buf in (o_buf, h_buf):
            assert bool((buf[:G] == -7.25).all()) and bool((buf[-G:] == -7.25).all()), wl.name
        r = compare_all(inp, out, hT)
        assert max(r["out"], r["hT"], r["chain_out"], r["chain_hT"]) <= TOL["bf16"], (wl.name, r)


def test_deterministic():
    inp = synth.generate(synth.custom(name="det", seed=34, B=2, T=300, H=4, dk=128, dv=128,
                                      dtype="bf16", chunk=64, h0_std=0.1))
    d = device_inputs(inp)
    o1, h1 = run_hip(inp, d=d)
    o2, h2 = run_hip(inp, d=d)
    assert torch.equal(_bits(o1), _bits(o2)) and torch.equal(_bits(h1), _bits(h2))


def test_hT_may_alias_h0():
    inp = synth.generate(synth.custom(name="alias", seed=35, B=2, T=130, H=2, dk=64, dv=64,
                                      dtype="bf16", chunk=64, h0_std=0.5))
    d = device_inputs(inp)
    o1, h1 = run_hip(inp, d=d)
    state = d["h0"].clone()
    d["h0"] = state
    o2, h2 = run_hip(inp, d=d, hT=state)
    assert h2.data_ptr() == state.data_ptr()
    assert torch.equal(_bits(o1), _bits(o2)) and torch.equal(_bits(h1), _bits(state))


def test_empty_inputs():
    # T == 0 (dense): hT = h0; zero-length packed sequences keep their h0.
    inp = synth.generate(synth.custom(name="empty", seed=36, B=2, T=0, H=2, dk=32, dv=32,
                                      dtype="bf16", chunk=64, h0_std=0.5))
    out, hT = run_hip(inp)
    assert out.numel() == 0
    assert torch.equal(hT, dev(inp.h0))
    inp = synth.generate(synth.custom(name="empty2", seed=37, H=2, dk=32, dv=32, dtype="bf16",
                                      chunk=64, seq_lens=[0, 0, 5]))
    d = device_inputs(inp)
    d["h0"] = torch.randn(3, 2, 32, 32, device="cuda")
    out, hT = run_hip(inp, d=d)
    assert torch.equal(hT[:2], d["h0"][:2])


def test_rejects_bad_args_without_launch():
    import gated_deltanet_recurrence_delta_amd as gdn

    inp = synth.generate(synth.custom(name="bad", seed=38, B=1, T=8, H=1, dk=32, dv=32,
                                      dtype="bf16", chunk=64))
    d = device_inputs(inp)
    with pytest.raises(gdn.GdnError):
        gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=16)


# ---------------------------------------------------------- sequence segments
# Dense bf16 batches with fewer workgroups than CUs run each sequence as
# several segments; a segment starts from a zero state far enough back that
# the transitions in between shrink any state by e^-40 (or at the sequence
# start).  These shapes have 8 or 16 workgroups and 16-32 chunks per
# sequence, so they are cut into 2-4 segments.

@pytest.mark.parametrize("kind", ["default_decay", "slow_decay", "no_decay", "long_keys"])
def test_segmented_sequences(kind):
    g_mean = {"default_decay": 0.0, "slow_decay": -4.0, "no_decay": 0.0, "long_keys": 0.0}[kind]
    wl = synth.custom(name=f"seg_{kind}", seed=40, B=1, T=2048, H=2, dk=128, dv=128, dtype="bf16",
                      chunk=64, h0_std=0.3, g_mean=g_mean)
    inp = synth.generate(wl)
    if kind == "no_decay":
        inp = dataclasses.replace(inp, g=np.zeros_like(inp.g))
    if kind == "long_keys":
        # |k| = 1.5 and beta near 1: the transitions can stretch the state
        # (|1 - beta |k|^2| > 1), which the segment start must account for
        k = synth.bf16_bits_to_f32(inp.k) * 1.5
        inp = dataclasses.replace(inp, k=synth.f32_to_bf16_bits(k),
                                  beta=np.clip(inp.beta + 0.4, 0, 1).astype(np.float32))
    _check(inp)


def test_segmented_small_state():
    inp = synth.generate(synth.custom(name="seg_small", seed=41, B=2, T=1024, H=4, dk=32, dv=32,
                                      dtype="bf16", chunk=64, h0_std=0.2))
    _check(inp)


def test_segmented_deterministic_and_alias_fallback():
    inp = synth.generate(synth.custom(name="seg_det", seed=42, B=1, T=1536, H=2, dk=128, dv=128,
                                      dtype="bf16", chunk=64, h0_std=0.3, g_mean=-3.0))
    o1, h1 = run_hip(inp)
    o2, h2 = run_hip(inp)
    assert torch.equal(_bits(o1), _bits(o2)) and torch.equal(_bits(h1), _bits(h2))
    # hT aliasing h0 runs unsegmented; it still matches the oracle
    d = device_inputs(inp)
    state = d["h0"].clone()
    d["h0"] = state
    o3, h3 = run_hip(inp, d=d, hT=state)
    eo, eh = compare(inp, o3, state)
    assert eo <= 2e-2 and eh <= 2e-2, (eo, eh)


def test_segmented_single_sequence_matches_packed():
    """A long sequence run alone and the same sequence inside a packed batch
    are cut into the same segments (the cut depends on the sequence alone),
    so their results agree bit for bit; both match the oracle."""
    lens = [2048, 300]
    wl = synth.custom(name="seg_vs_packed", seed=43, H=2, dk=128, dv=128, dtype="bf16", chunk=64,
                      seq_lens=lens)
    inp = synth.generate(wl)
    d = device_inputs(inp)
    h0 = torch.randn(len(lens), 2, 128, 128, device="cuda") * 0.1
    d["h0"] = h0
    out, hT = run_hip(inp, d=d)
    o1, h1 = run_hip(inp, d=_alone(d, 0, 2048, h0[:1].contiguous()))
    assert torch.equal(_bits(out[:2048]), _bits(o1[0]))
    assert torch.equal(_bits(hT[0]), _bits(h1[0]))
    eo, eh = compare(dataclasses.replace(inp, h0=h0.cpu().numpy()), out, hT)
    assert eo <= 2e-2 and eh <= 2e-2, (eo, eh)


@pytest.mark.parametrize("dk,dv,chunk", [(64, 64, 64), (128, 128, 32), (32, 128, 64)])
def test_segmented_other_shapes(dk, dv, chunk):
    inp = synth.generate(synth.custom(name=f"seg_{dk}_{dv}_{chunk}", seed=44, B=1, T=1600, H=3,
                                      dk=dk, dv=dv, dtype="bf16", chunk=chunk, h0_std=0.2,
                                      g_mean=-2.0))
    _check(inp)
