"""GPU parity of the diagonal-decay additive recurrence (both entry points)
against the FP64 oracle, element by element on the same stored inputs."""
import dataclasses

import numpy as np
import pytest

import synth.diag as sd
from oracle import diag as odiag
from oracle import rel_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _dev(x):
    import torch

    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _host(t):
    import torch

    return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy().astype(np.float64)


def run(inp, form="chunked", **kw):
    import torch

    import gated_deltanet_recurrence_delta_amd as gdn

    d = {k: _dev(getattr(inp, k)) for k in ("v", "b", "c", "g", "A_log", "Dskip", "gate", "h0",
                                            "cu_seqlens")}
    f = gdn.diag_fwd if form == "chunked" else gdn.diag_fwd_recurrent
    out, hT = f(d["v"], d["b"], d["c"], d["g"], d["A_log"], D=d["Dskip"], gate=d["gate"],
                h0=d["h0"], cu_seqlens=d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return out, hT


def oracle(inp):
    f = lambda n: inp.as_f64(n)
    return odiag.diag_fwd_seq(f("v"), f("b"), f("c"), f("g"), f("A_log"), f("h0"),
                              inp.cu_seqlens, f("Dskip"), f("gate"))


def check(inp, form, tol=None):
    out, hT = run(inp, form)
    o_ref, h_ref = oracle(inp)
    eo, eh = rel_err(_host(out), o_ref), rel_err(_host(hT), h_ref)
    tol = tol or TOL[inp.wl.dtype]
    print(f"{inp.wl.name} {form}: rel err out {eo:.2e} hT {eh:.2e}", flush=True)
    assert eo <= tol and eh <= tol, (eo, eh)
    return out, hT


# ---------------------------------------------------------------- recurrent

@pytest.mark.parametrize("S,D", [(32, 32), (16, 32), (64, 16), (128, 64), (32, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_recurrent_shapes(S, D, dtype):
    inp = sd.generate(sd.custom(f"rec_{S}_{D}_{dtype}", seed=S + D, B=2, T=29, H=3, S=S, D=D,
                                dtype=dtype, h0_std=0.3))
    check(inp, "recurrent")


def test_recurrent_without_epilogue_or_state():
    inp = sd.generate(sd.custom("rec_plain", seed=3, B=3, T=40, H=2, dtype="f32", epilogue=False))
    check(inp, "recurrent")


def test_recurrent_packed_with_empty_sequences():
    inp = sd.generate(sd.custom("rec_packed", seed=4, H=3, dtype="f32", h0_std=0.2,
                                seq_lens=[5, 0, 17, 1, 0, 33]))
    check(inp, "recurrent")


def test_recurrent_decode_step():
    inp = sd.generate(sd.custom("rec_decode", seed=5, B=64, T=1, H=40, dtype="bf16", h0_std=0.2))
    check(inp, "recurrent")


# ----------------------------------------------------------------- chunked

@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 200, 700])
def test_chunked_lengths(T):
    inp = sd.generate(sd.custom(f"chunk_T{T}", seed=T, B=2, T=T, H=3, dtype="bf16", h0_std=0.3))
    check(inp, "chunked")


def test_chunked_without_epilogue_or_state():
    inp = sd.generate(sd.custom("chunk_plain", seed=8, B=2, T=300, H=2, dtype="bf16",
                                epilogue=False))
    check(inp, "chunked")


def test_chunked_packed_with_empty_sequences():
    inp = sd.generate(sd.custom("chunk_packed", seed=9, H=4, dtype="bf16", h0_std=0.2,
                                seq_lens=[70, 0, 130, 1, 64, 0, 600, 33]))
    check(inp, "chunked")


@pytest.mark.parametrize("lo,hi", [(-6.0, 0.0), (3.0, 6.0), (-3.0, 4.5)])
def test_chunked_decay_extremes(lo, hi):
    """Rows that barely decay, rows whose decay underflows within a token or
    two (A = -400 per unit of g), and a mix within one head."""
    inp = sd.generate(sd.custom(f"chunk_decay_{lo}_{hi}", seed=11, B=2, T=260, H=3, dtype="bf16",
                                h0_std=0.3))
    rng = np.random.default_rng(12)
    inp = dataclasses.replace(inp, A_log=rng.uniform(lo, hi, size=inp.A_log.shape).astype(np.float32))
    check(inp, "chunked")


def test_chunked_zero_gate_is_linear_attention():
    inp = sd.generate(sd.custom("chunk_g0", seed=13, B=1, T=200, H=2, dtype="bf16", h0_std=0.3))
    inp = dataclasses.replace(inp, g=np.zeros_like(inp.g))
    check(inp, "chunked")


def test_chunked_agrees_with_recurrent():
    inp = sd.generate(sd.custom("chunk_vs_rec", seed=14, B=2, T=333, H=5, dtype="bf16",
                                h0_std=0.2))
    o1, h1 = run(inp, "chunked")
    o2, h2 = run(inp, "recurrent")
    eo = rel_err(_host(o1), _host(o2))
    eh = rel_err(_host(h1), _host(h2))
    print(f"chunked vs recurrent: out {eo:.2e} hT {eh:.2e}", flush=True)
    assert eo <= 2e-2 and eh <= 2e-2


def test_chunked_deterministic_and_in_place_state():
    import torch

    import gated_deltanet_recurrence_delta_amd as gdn

    inp = sd.generate(sd.custom("chunk_det", seed=15, B=2, T=257, H=3, dtype="bf16", h0_std=0.3))
    o1, h1 = run(inp, "chunked")
    o2, h2 = run(inp, "chunked")
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    d = {k: _dev(getattr(inp, k)) for k in ("v", "b", "c", "g", "A_log", "Dskip", "gate", "h0")}
    st = d["h0"].clone()
    o3, h3 = gdn.diag_fwd(d["v"], d["b"], d["c"], d["g"], d["A_log"], D=d["Dskip"],
                          gate=d["gate"], h0=st, hT=st)
    torch.cuda.synchronize()
    assert torch.equal(o3, o1) and torch.equal(st, h1)


def test_chunked_split_composes():
    """Two calls over [0, t) and [t, T), the second starting from the first's
    final state, agree with one call within the bf16 tolerance."""
    import torch

    import gated_deltanet_recurrence_delta_amd as gdn

    inp = sd.generate(sd.custom("chunk_split", seed=16, B=2, T=300, H=3, dtype="bf16", h0_std=0.3))
    d = {k: _dev(getattr(inp, k)) for k in ("v", "b", "c", "g", "A_log", "Dskip", "gate", "h0")}
    full_o, full_h = gdn.diag_fwd(d["v"], d["b"], d["c"], d["g"], d["A_log"], D=d["Dskip"],
                                  gate=d["gate"], h0=d["h0"])
    cut = 100
    part = lambda x, sl: x[:, sl].contiguous()
    o1, h1 = gdn.diag_fwd(*(part(d[k], slice(0, cut)) for k in ("v", "b", "c", "g")), d["A_log"],
                          D=d["Dskip"], gate=part(d["gate"], slice(0, cut)), h0=d["h0"])
    o2, h2 = gdn.diag_fwd(*(part(d[k], slice(cut, None)) for k in ("v", "b", "c", "g")),
                          d["A_log"], D=d["Dskip"], gate=part(d["gate"], slice(cut, None)), h0=h1)
    torch.cuda.synchronize()
    eo = rel_err(_host(torch.cat([o1, o2], dim=1)), _host(full_o))
    eh = rel_err(_host(h2), _host(full_h))
    assert eo <= 2e-2 and eh <= 2e-2, (eo, eh)


def test_chunked_empty_inputs():
    import torch

    import gated_deltanet_recurrence_delta_amd as gdn

    H, S, D = 3, 32, 32
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    f = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda")
    h0 = torch.randn(2, H, S, D, device="cuda")
    out, hT = gdn.diag_fwd(z(2, 0, H, D), z(2, 0, H, S), z(2, 0, H, S), f(2, 0, H), f(H, S), h0=h0)
    torch.cuda.synchronize()
    assert out.numel() == 0 and torch.equal(hT, h0)


def test_chunked_rejects_unsupported():
    import gated_deltanet_recurrence_delta_amd as gdn

    inp = sd.generate(sd.custom("chunk_f32", seed=17, B=1, T=20, H=2, dtype="f32"))
    with pytest.raises(gdn.GdnError):
        run(inp, "chunked")


def test_chunked_hymo_workload_sampled():
    """The HyMo layer's shape (B=4, T=4096, H=40, S=D=32) in the launch the
    benchmark times; the oracle evaluates one whole batch row (40 chains)."""
    inp = sd.generate(sd.WORKLOADS["hymo"])
    out, hT = run(inp, "chunked")
    b = 3
    sub = dataclasses.replace(
        inp, v=inp.v[b:b + 1], b=inp.b[b:b + 1], c=inp.c[b:b + 1], g=inp.g[b:b + 1],
        gate=inp.gate[b:b + 1], h0=None if inp.h0 is None else inp.h0[b:b + 1])
    o_ref, h_ref = oracle(sub)
    eo = rel_err(_host(out)[b:b + 1], o_ref)
    eh = rel_err(_host(hT)[b:b + 1], h_ref)
    print(f"hymo batch row {b}: rel err out {eo:.2e} hT {eh:.2e}", flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]


@pytest.mark.parametrize("which", ["skip_only", "gate_only"])
@pytest.mark.parametrize("form", ["chunked", "recurrent"])
def test_epilogue_factors_separately(which, form):
    inp = sd.generate(sd.custom(f"epi_{which}_{form}", seed=21, B=2, T=90, H=3, dtype="bf16",
                                h0_std=0.2))
    inp = dataclasses.replace(inp, gate=None) if which == "skip_only" else dataclasses.replace(inp, Dskip=None)
    check(inp, form)


def test_chunked_many_heads_one_sequence():
    """One sequence, 96 heads: more chains than one XCD's share, B = 1."""
    inp = sd.generate(sd.custom("chunk_h96", seed=22, B=1, T=150, H=96, dtype="bf16", h0_std=0.2))
    check(inp, "chunked")


def test_chunked_packed_ragged_lengths():
    """Packed lengths off the 16- and 64-token grids, one of them spanning
    more chunks than the workgroup has waves (9 x 64 + 5 tokens)."""
    lens = [3, 17, 31, 47, 64 * 9 + 5, 80, 2, 0, 129]
    inp = sd.generate(sd.custom("chunk_ragged", seed=23, H=2, dtype="bf16", h0_std=0.2,
                                seq_lens=lens))
    check(inp, "chunked")


def test_recurrent_packed_equals_per_sequence_bitwise():
    import torch

    lens = [9, 0, 21, 4]
    inp = sd.generate(sd.custom("rec_bitwise", seed=24, H=3, dtype="f32", h0_std=0.3,
                                seq_lens=lens))
    out, hT = run(inp, "recurrent")
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        s, e = int(cu[n]), int(cu[n + 1])
        sub = dataclasses.replace(
            inp, wl=sd.custom("one", seed=0, B=1, T=e - s, H=3, dtype="f32"),
            v=inp.v[None, s:e], b=inp.b[None, s:e], c=inp.c[None, s:e], g=inp.g[None, s:e],
            gate=inp.gate[None, s:e], h0=inp.h0[n:n + 1], cu_seqlens=None)
        o1, h1 = run(sub, "recurrent")
        assert torch.equal(o1[0], out[s:e]) and torch.equal(h1[0], hT[n])


def test_chunked_packed_equals_per_sequence_bitwise():
    """Each sequence's slice of a packed run equals that sequence run alone,
    both packed by itself (cu_seqlens = [0, L]) and, where the dense batch
    is too short to split into segments, as a dense B = 1 batch."""
    import torch

    lens = [70, 0, 130, 1, 64 * 9 + 5, 33, 64]
    inp = sd.generate(sd.custom("chunk_bitwise", seed=29, H=3, dtype="bf16", h0_std=0.3,
                                seq_lens=lens))
    out, hT = run(inp, "chunked")
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        s, e = int(cu[n]), int(cu[n + 1])
        packed = dataclasses.replace(
            inp, wl=sd.custom("one", seed=0, H=3, dtype="bf16", seq_lens=[e - s]),
            v=inp.v[s:e], b=inp.b[s:e], c=inp.c[s:e], g=inp.g[s:e], gate=inp.gate[s:e],
            h0=inp.h0[n:n + 1], cu_seqlens=np.array([0, e - s], dtype=np.int32))
        o1, h1 = run(packed, "chunked")
        assert torch.equal(o1, out[s:e]) and torch.equal(h1[0], hT[n]), n
        if (e - s + 63) // 64 < 8:  # fewer than 8 chunks: never split
            dense = dataclasses.replace(
                packed, wl=sd.custom("one", seed=0, B=1, T=e - s, H=3, dtype="bf16"),
                v=inp.v[None, s:e], b=inp.b[None, s:e], c=inp.c[None, s:e], g=inp.g[None, s:e],
                gate=inp.gate[None, s:e], cu_seqlens=None)
            o2, h2 = run(dense, "chunked")
            assert torch.equal(o2[0], out[s:e]) and torch.equal(h2[0], hT[n]), n


# Dense batches with fewer chains than two workgroups per CU run each
# sequence as segments that start from a zero state where the decay since
# then is below e^-40 (or at the sequence start).  Two chains and 32 chunks
# give 8 segments of 4 chunks.
@pytest.mark.parametrize("decay", ["default", "slow", "none", "mixed"])
def test_chunked_segments(decay):
    inp = sd.generate(sd.custom(f"chunk_seg_{decay}", seed=25, B=1, T=2048, H=2, dtype="bf16",
                                h0_std=0.3))
    rng = np.random.default_rng(26)
    if decay == "slow":
        inp = dataclasses.replace(inp, A_log=np.full_like(inp.A_log, -4.0))
    elif decay == "none":
        inp = dataclasses.replace(inp, g=np.zeros_like(inp.g))
    elif decay == "mixed":  # one row barely decays, the others fast
        a = rng.uniform(1.0, 3.0, size=inp.A_log.shape).astype(np.float32)
        a[:, 5] = -7.0
        inp = dataclasses.replace(inp, A_log=a)
    check(inp, "chunked")


# Six chains of 21 chunks, the last one partial, each with its own initial
# state: 5 segments of 5 chunks per sequence, the last one ragged.
@pytest.mark.parametrize("decay", ["default", "slow", "none"])
def test_chunked_segments_ragged_with_state(decay):
    inp = sd.generate(sd.custom(f"chunk_win_{decay}", seed=28, B=2, T=1307, H=3, dtype="bf16",
                                h0_std=0.3))
    if decay == "slow":
        inp = dataclasses.replace(inp, A_log=np.full_like(inp.A_log, -4.0))
    elif decay == "none":
        inp = dataclasses.replace(inp, g=np.zeros_like(inp.g))
    check(inp, "chunked")


def test_chunked_segments_hymo_heads_alias_fallback():
    """hT aliasing h0 turns segments off; the result still matches."""
    import torch

    import gated_deltanet_recurrence_delta_amd as gdn

    inp = sd.generate(sd.custom("chunk_seg_alias", seed=27, B=1, T=1024, H=3, dtype="bf16",
                                h0_std=0.3))
    d = {k: _dev(getattr(inp, k)) for k in ("v", "b", "c", "g", "A_log", "Dskip", "gate", "h0")}
    st = d["h0"].clone()
    out, _ = gdn.diag_fwd(d["v"], d["b"], d["c"], d["g"], d["A_log"], D=d["Dskip"],
                          gate=d["gate"], h0=st, hT=st)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle(inp)
    assert rel_err(_host(out), o_ref) <= 2e-2 and rel_err(_host(st), h_ref) <= 2e-2
