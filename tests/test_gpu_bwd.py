"""Backward entry point (gdn_bwd) vs the FP64 reverse-sweep oracle
(``oracle.bwd``), element by element, through the C ABI.

Every gradient (dq, dk, dv, dg, dbeta, dh0) is compared in the infinity
norm relative to the oracle's largest entry of the same tensor.  The kernels
compute in fp32 from the stored inputs, so float32 storage is held to 1e-4
and bfloat16 storage to 2e-2 (the token gradients are rounded to bfloat16 on
store).  Sizes span several 32-token chunks with ragged tails, both storage
dtypes, every supported head size, packed batches with empty and one-token
sequences, and the degenerate decays (none, and strong).
"""
import numpy as np
import pytest

import synth
from hip_case import TOL, dev, host_f64
from oracle.bwd import bwd_seq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _run(inp, og, want_dh0=True, workspace=None):
    import gated_deltanet_recurrence_delta_amd as gdn

    grads = gdn.bwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                    dev(og.dout), h0=dev(inp.h0), cu_seqlens=dev(inp.cu_seqlens),
                    dhT=dev(og.dhT), want_dh0=want_dh0, workspace=workspace)
    torch.cuda.synchronize()
    return grads


def _oracle(inp, og):
    return bwd_seq(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.as_f64("g"),
                   inp.as_f64("beta"), inp.as_f64("h0"), inp.cu_seqlens,
                   og.as_f64("dout"), og.as_f64("dhT"))


def _rel(a, b):
    if b.size == 0:
        return 0.0
    den = float(np.max(np.abs(b)))
    num = float(np.max(np.abs(a - b)))
    return 0.0 if num == 0.0 else num / max(den, 1e-30)


def _check(inp, og, tol=None, label=""):
    grads = _run(inp, og)
    ref = _oracle(inp, og)
    tol = tol if tol is not None else TOL[inp.wl.dtype]
    errs = {n: _rel(host_f64(grads[n]), ref[n]) for n in NAMES}
    print(f"{label or inp.wl.name}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items())
          + f" (tol {tol:g})", flush=True)
    for n, e in errs.items():
        assert e <= tol, (n, e)
    return grads


CASES = [
    # (dtype, B, T, H, dk, dv, h0_std, dhT_std, g_mean)
    ("f32", 2, 75, 2, 32, 32, 0.3, 1.0, 0.0),
    ("f32", 1, 100, 2, 64, 128, 0.0, 0.0, 0.0),
    ("f32", 1, 64, 1, 128, 64, 0.3, 0.5, 0.0),
    ("f32", 2, 33, 3, 128, 128, 0.2, 1.0, -2.0),
    ("f32", 1, 1, 2, 64, 64, 0.5, 1.0, 0.0),
    ("f32", 1, 31, 2, 32, 128, 0.0, 1.0, 0.0),
    ("bf16", 2, 97, 2, 128, 128, 0.3, 1.0, 0.0),
    ("bf16", 1, 130, 2, 32, 64, 0.0, 1.0, 0.0),
    ("bf16", 1, 64, 3, 64, 32, 0.2, 0.0, 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_shapes(case):
    dtype, B, T, H, dk, dv, h0, dh, gm = case
    wl = synth.custom(name="bwd", seed=700 + CASES.index(case), B=B, T=T, H=H, dk=dk, dv=dv,
                      dtype=dtype, h0_std=h0, g_mean=gm)
    inp = synth.generate(wl)
    _check(inp, synth.output_grads(inp, 800 + CASES.index(case), dh))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_packed(dtype):
    """Packed sequences with an empty one, a one-token one, exact and ragged
    multiples of the chunk."""
    wl = synth.custom(name="bwd_packed", seed=710, H=2, dk=64, dv=32, dtype=dtype,
                      h0_std=0.3, seq_lens=(33, 0, 1, 70, 32, 5))
    inp = synth.generate(wl)
    _check(inp, synth.output_grads(inp, 810))


def test_packed_wide():
    wl = synth.custom(name="bwd_packed_wide", seed=711, H=2, dk=128, dv=128, dtype="bf16",
                      h0_std=0.2, seq_lens=(40, 95, 0, 64))
    inp = synth.generate(wl)
    _check(inp, synth.output_grads(inp, 811))


def test_no_decay():
    """g = 0: nothing decays, every exponential factor is 1."""
    wl = synth.custom(name="bwd_g0", seed=712, B=1, T=70, H=2, dk=32, dv=32, dtype="f32",
                      h0_std=0.3)
    inp = synth.generate(wl)
    inp.g[...] = 0.0
    _check(inp, synth.output_grads(inp, 812))


def test_strong_decay():
    """g = -30 on every token: each token forgets all earlier ones (the
    exponential factors underflow to zero)."""
    wl = synth.custom(name="bwd_gneg", seed=713, B=1, T=50, H=2, dk=32, dv=64, dtype="f32",
                      h0_std=0.3)
    inp = synth.generate(wl)
    inp.g[...] = -30.0
    _check(inp, synth.output_grads(inp, 813))


def test_empty_sequences():
    """T = 0: no token gradients; dh0 = dhT."""
    wl = synth.custom(name="bwd_empty", seed=714, B=2, T=0, H=2, dk=32, dv=32, dtype="f32",
                      h0_std=0.3)
    inp = synth.generate(wl)
    og = synth.output_grads(inp, 814)
    grads = _run(inp, og)
    assert grads["dq"].numel() == 0
    assert torch.equal(grads["dh0"].cpu(), torch.from_numpy(og.dhT))


def test_packed_equals_per_sequence_bitwise():
    """Each sequence of a packed call gets exactly the gradients of a call
    with that sequence alone (same chunking, same arithmetic)."""
    lens = (45, 7, 64)
    wl = synth.custom(name="bwd_pps", seed=715, H=2, dk=64, dv=64, dtype="bf16", h0_std=0.3,
                      seq_lens=lens)
    inp = synth.generate(wl)
    og = synth.output_grads(inp, 815)
    grads = _run(inp, og)
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        s, e = int(cu[n]), int(cu[n + 1])
        one = synth.Inputs(wl=wl, q=inp.q[s:e][None], k=inp.k[s:e][None], v=inp.v[s:e][None],
                           g=inp.g[s:e][None], beta=inp.beta[s:e][None],
                           h0=inp.h0[n:n + 1], cu_seqlens=None)
        one_og = synth.OutputGrads(dout=og.dout[s:e][None], dhT=og.dhT[n:n + 1])
        g1 = _run(one, one_og)
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            assert torch.equal(grads[name][s:e], g1[name][0]), (n, name)
        assert torch.equal(grads["dh0"][n], g1["dh0"][0]), n


def test_deterministic_and_optional_dh0():
    wl = synth.custom(name="bwd_det", seed=716, B=2, T=90, H=2, dk=128, dv=64, dtype="bf16",
                      h0_std=0.2)
    inp = synth.generate(wl)
    og = synth.output_grads(inp, 816)
    a = _run(inp, og)
    b = _run(inp, og, want_dh0=False)
    assert b["dh0"] is None
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert torch.equal(a[name], b[name]), name


def test_workspace_reuse():
    """A caller-held workspace, used for a larger and then a smaller call,
    gives the same results as a fresh one (nothing is carried over)."""
    import gated_deltanet_recurrence_delta_amd as gdn

    big = synth.generate(synth.custom(name="bwd_ws1", seed=717, B=2, T=80, H=2, dk=64, dv=64,
                                      dtype="f32", h0_std=0.3))
    small = synth.generate(synth.custom(name="bwd_ws2", seed=718, B=1, T=37, H=2, dk=64, dv=64,
                                        dtype="f32", h0_std=0.3))
    need = gdn.gdn_bwd_workspace_size(2, 80, 2, 64, 64, 0)
    ws = torch.full((need,), 0x7f, dtype=torch.uint8, device="cuda")
    og_b, og_s = synth.output_grads(big, 817), synth.output_grads(small, 818)
    ref = _run(small, og_s)
    _run(big, og_b, workspace=ws)
    again = _run(small, og_s, workspace=ws)
    for name in NAMES:
        assert torch.equal(ref[name], again[name]), name


def test_wide_head_shape_two_chains():
    """The wide_head shape (dk = dv = 128, bf16, nonzero h0) at 2,048 tokens,
    two chains, every gradient against the oracle."""
    wl = synth.custom(name="bwd_wide", seed=719, B=1, T=2048, H=2, dk=128, dv=128,
                      dtype="bf16", h0_std=0.02)
    inp = synth.generate(wl)
    _check(inp, synth.output_grads(inp, 819))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_long_sequence(dtype):
    """4,096 tokens (128 chunks through both serial sweeps) with slow decay and
    a nonzero initial state: rounding must not build up along the chain."""
    wl = synth.custom(name="bwd_long", seed=720, B=1, T=4096, H=2, dk=32, dv=32, dtype=dtype,
                      h0_std=0.3, g_mean=-4.0)
    inp = synth.generate(wl)
    _check(inp, synth.output_grads(inp, 820))


@pytest.mark.parametrize("kind", ["fast_decay", "slow_decay", "no_decay"])
def test_segmented_sweeps(kind):
    """One long chain with few (chain, tile) workgroups: both serial sweeps
    run as segments with halos (2,048 tokens = 64 chunks in 8 segments).
    With no decay every halo reaches the sequence end, so the result is exact
    up to rounding; with decay the halos stop where the transition-norm
    product is below e^-40."""
    g_mean = {"fast_decay": 0.0, "slow_decay": -4.0, "no_decay": 0.0}[kind]
    wl = synth.custom(name=f"bwd_seg_{kind}", seed=721, B=1, T=2048, H=1, dk=32, dv=32,
                      dtype="f32", h0_std=0.3, g_mean=g_mean)
    inp = synth.generate(wl)
    if kind == "no_decay":
        inp.g[...] = 0.0
    og = synth.output_grads(inp, 821)
    a = _check(inp, og, label=wl.name)
    b = _run(inp, og)
    for name in NAMES:
        assert torch.equal(a[name], b[name]), name  # deterministic


def test_segmented_bf16_wide():
    """Segments at d = 128, bf16: one chain, 1,024 tokens (32 chunks, 8 tiles
    of 16 columns -> 4 segments)."""
    wl = synth.custom(name="bwd_seg_wide", seed=722, B=1, T=1024, H=1, dk=128, dv=128,
                      dtype="bf16", h0_std=0.02, g_mean=-2.0)
    inp = synth.generate(wl)
    _check(inp, synth.output_grads(inp, 822))


@pytest.mark.parametrize("name", ["wide_head", "small_state"])
def test_full_workload_sampled_chains(name):
    """The full workload (wide_head: B=4 H=16 T=4096 d=128 bf16; small_state:
    B=8 H=16 T=4096 d=32, whose sweeps run in segments) in one call, in the
    configuration bench.py --pass bwd times; the oracle checks two chains,
    (first sequence, first head) and (last, last), every gradient."""
    wl = synth.WORKLOADS[name]
    inp = synth.generate(wl)
    og = synth.output_grads(inp, 1000 + wl.seed)
    grads = _run(inp, og)
    tol = TOL[wl.dtype]
    for b, h in ((0, 0), (wl.B - 1, wl.H - 1)):
        cut = lambda x: None if x is None else x[b:b + 1, :, h:h + 1]
        ref = bwd_seq(*(cut(inp.as_f64(n)) for n in ("q", "k", "v", "g", "beta")),
                      None if inp.h0 is None else inp.as_f64("h0")[b:b + 1, h:h + 1], None,
                      cut(og.as_f64("dout")),
                      None if og.dhT is None else og.as_f64("dhT")[b:b + 1, h:h + 1])
        errs = {n: _rel(host_f64(grads[n][b:b + 1, :, h:h + 1]), ref[n])
                for n in ("dq", "dk", "dv", "dg", "dbeta")}
        errs["dh0"] = _rel(host_f64(grads["dh0"][b:b + 1, h:h + 1]), ref["dh0"])
        print(f"{name} chain ({b},{h}): " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()),
              flush=True)
        for n, e in errs.items():
            assert e <= tol, (n, e)


def test_autograd_function():
    """gated_delta_rule as a torch autograd operation: a scalar loss built
    from out and hT back-propagates to every input (including h0) with the
    oracle's gradients of the same loss."""
    import gated_deltanet_recurrence_delta_amd as gdn

    wl = synth.custom(name="bwd_autograd", seed=723, B=2, T=70, H=2, dk=64, dv=32,
                      dtype="f32", h0_std=0.3)
    inp = synth.generate(wl)
    og = synth.output_grads(inp, 823)
    x = {n: dev(getattr(inp, n)).requires_grad_(True) for n in ("q", "k", "v", "g", "beta", "h0")}
    out, hT = gdn.gated_delta_rule(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    loss = (out * dev(og.dout)).sum() + (hT * dev(og.dhT)).sum()
    loss.backward()
    ref = _oracle(inp, og)
    for n, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                     ("h0", "dh0")):
        e = _rel(host_f64(x[n].grad), ref[gname])
        assert e <= 1e-4, (gname, e)


TRAIN_CASES = [
    # (B, T, H, seq_lens, h0_std): one chain cut into two segments (21 chunks),
    # and a packed batch with an empty, a short and a cut sequence
    (2, 1300, 3, None, 0.2),
    (None, None, 2, (40, 95, 0, 64, 1300), 0.2),
]


@pytest.mark.parametrize("case", TRAIN_CASES, ids=["dense", "packed"])
def test_training_forward_records_bitwise(case):
    """fwd_train's out and hT equal fwd's bit for bit, and the backward from
    its records (gdn_bwd_saved) equals the backward that recomputes them
    (gdn_bwd) bit for bit, every gradient; both agree with the oracle."""
    import gated_deltanet_recurrence_delta_amd as gdn

    B, T, H, lens, h0s = case
    if lens is None:
        wl = synth.custom(name="train_dense", seed=730, B=B, T=T, H=H, dk=128, dv=128, dtype="bf16",
                          h0_std=h0s, g_mean=-2.0)
    else:
        wl = synth.custom(name="train_packed", seed=731, H=H, dk=128, dv=128, dtype="bf16",
                          h0_std=h0s, g_mean=-2.0, seq_lens=lens)
    inp = synth.generate(wl)
    og = synth.output_grads(inp, 830)
    d = {n: dev(getattr(inp, n)) for n in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")}
    out1, hT1 = gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"])
    out2, hT2, ws = gdn.fwd_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(hT1.view(torch.int32), hT2.view(torch.int32))
    g1 = _run(inp, og)
    g2 = gdn.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dev(og.dout), h0=d["h0"],
                 cu_seqlens=d["cu_seqlens"], dhT=dev(og.dhT), workspace=ws, saved=True)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(g1[n], g2[n]), n
    ref = _oracle(inp, og)
    for n in NAMES:
        e = _rel(host_f64(g2[n]), ref[n])
        assert e <= TOL["bf16"], (n, e)


def test_autograd_function_full_width():
    """gated_delta_rule at bf16 with dk = dv = 128 runs gdn_fwd_train and
    gdn_bwd_saved: its gradients equal gdn.bwd's (which recomputes the
    states) bit for bit."""
    import gated_deltanet_recurrence_delta_amd as gdn

    wl = synth.custom(name="bwd_autograd_wide", seed=724, B=2, T=300, H=2, dk=128, dv=128,
                      dtype="bf16", h0_std=0.2)
    inp = synth.generate(wl)
    og = synth.output_grads(inp, 824)
    x = {n: dev(getattr(inp, n)).requires_grad_(True) for n in ("q", "k", "v", "g", "beta", "h0")}
    out, hT = gdn.gated_delta_rule(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    loss = (out.float() * dev(og.dout).float()).sum() + (hT * dev(og.dhT)).sum()
    loss.backward()
    ref = _run(inp, og)
    for n, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                     ("h0", "dh0")):
        assert torch.equal(x[n].grad, ref[gname]), gname


@pytest.mark.parametrize("name", ["wide_head", "long_context"])
def test_adjoint_identity_full_workload(name):
    """out and hT are jointly linear in (v, h0), so for any dout and dhT,
    <dout, out> + <dhT, hT> = <dv, v> + <dh0, h0>.  Checked with the GPU
    forward (gdn_fwd) and the GPU backward (gdn_bwd) on every chain of the
    full workload -- a property that holds at any size, no oracle needed.
    The two sides are sums of ~1e8 products of bf16 data; with rounding of
    random sign they agree to ~1e-6 of the sum of the terms' magnitudes,
    while a missing or sign-flipped term moves them by ~3e-4 of it."""
    import gated_deltanet_recurrence_delta_amd as gdn

    wl = synth.WORKLOADS[name]
    inp = synth.generate(wl)
    og = synth.output_grads(inp, 1100 + wl.seed)
    d = {n: dev(getattr(inp, n)) for n in ("q", "k", "v", "g", "beta", "h0")}
    h0 = d["h0"] if d["h0"] is not None else torch.zeros(
        (wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    out, hT = gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], h0, chunk=wl.chunk)
    grads = gdn.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dev(og.dout), h0=h0,
                    dhT=dev(og.dhT))
    torch.cuda.synchronize()
    f64 = lambda t: t.double()
    lhs = float((f64(dev(og.dout)) * f64(out)).sum() + (f64(dev(og.dhT)) * f64(hT)).sum())
    rhs = float((f64(grads["dv"]) * f64(d["v"])).sum() + (f64(grads["dh0"]) * f64(h0)).sum())
    scale = float((f64(dev(og.dout)).abs() * f64(out).abs()).sum()
                  + (f64(dev(og.dhT)).abs() * f64(hT).abs()).sum())
    print(f"{name}: <dout,out>+<dhT,hT> {lhs:.6e}  <dv,v>+<dh0,h0> {rhs:.6e}  "
          f"rel to sum |terms| {abs(lhs - rhs) / scale:.2e}", flush=True)
    assert abs(lhs - rhs) <= 5e-5 * scale


@pytest.mark.parametrize("T", [70, 200, 136])
def test_partial_last_chunk_slow_decay(T):
    """bf16 d = 128 (the 64-token full-width kernels) with a ragged last
    chunk and slow decay, so that every exit-decay factor w of the partial
    chunk is far from zero and each token's dg takes the w terms of all the
    tokens before it (a defect in how one lane's term reached the next
    showed here and not under the default decay)."""
    wl = synth.custom(name=f"bwd_tail{T}", seed=730 + T, B=2, T=T, H=2, dk=128, dv=128,
                      dtype="bf16", h0_std=0.3, g_mean=-4.0)
    inp = synth.generate(wl)
    _check(inp, synth.output_grads(inp, 830 + T))
