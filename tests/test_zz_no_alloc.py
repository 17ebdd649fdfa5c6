"""gdn_bwd_noalloc (the backward pass on the library's fixed per-GPU scratch)
against gdn_bwd with a caller-owned workspace, through the C ABI: two calls
in a row, the second on a smaller problem, each compared bit for bit with
gdn_bwd on the same inputs, and both within tolerance of the FP64 oracle."""
import numpy as np
import pytest

import synth
from hip_case import TOL, dev, host_f64
from oracle.bwd import bwd_seq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _noalloc(inp, og):
    import gated_deltanet_recurrence_delta_amd as gdn

    d = {n: dev(getattr(inp, n)) for n in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")}
    dout, dhT = dev(og.dout), dev(og.dhT)
    B = len(inp.cu_seqlens) - 1 if inp.cu_seqlens is not None else inp.wl.B
    T = int(inp.cu_seqlens[-1]) if inp.cu_seqlens is not None else inp.wl.T
    wl = inp.wl
    g = {"dq": torch.empty_like(d["q"]), "dk": torch.empty_like(d["k"]),
         "dv": torch.empty_like(d["v"]), "dg": torch.empty_like(d["g"]),
         "dbeta": torch.empty_like(d["beta"]),
         "dh0": torch.empty(B, wl.H, wl.dk, wl.dv, device="cuda")}
    ptr = lambda t: 0 if t is None else t.data_ptr()
    dtype = gdn.GDN_BF16 if wl.dtype == "bf16" else gdn.GDN_F32
    rc = gdn.gdn_bwd_noalloc(ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["g"]), ptr(d["beta"]),
                             ptr(d["h0"]), ptr(d["cu_seqlens"]), ptr(dout), ptr(dhT),
                             ptr(g["dq"]), ptr(g["dk"]), ptr(g["dv"]), ptr(g["dg"]),
                             ptr(g["dbeta"]), ptr(g["dh0"]), B, T, wl.H, wl.dk, wl.dv,
                             torch.cuda.current_stream().cuda_stream, dtype)
    assert rc == 0, gdn.strerror(rc)
    torch.cuda.synchronize()
    return g


def _with_workspace(inp, og):
    import gated_deltanet_recurrence_delta_amd as gdn

    g = gdn.bwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(og.dout),
                h0=dev(inp.h0), cu_seqlens=dev(inp.cu_seqlens), dhT=dev(og.dhT))
    torch.cuda.synchronize()
    return g


def _rel(a, b):
    den = float(np.max(np.abs(b))) if b.size else 0.0
    num = float(np.max(np.abs(a - b))) if b.size else 0.0
    return 0.0 if num == 0.0 else num / max(den, 1e-30)


def test_noalloc_matches_workspace_entry_point_twice():
    cases = [synth.custom(name="na1", seed=61, B=2, T=200, H=2, dk=128, dv=128, dtype="bf16",
                          h0_std=0.3),
             synth.custom(name="na2", seed=62, H=2, dk=64, dv=64, dtype="bf16",
                          seq_lens=[70, 0, 33])]
    for wl in cases:
        inp = synth.generate(wl)
        og = synth.output_grads(inp, 63)
        got = _noalloc(inp, og)
        want = _with_workspace(inp, og)
        for n in NAMES:
            assert torch.equal(_bits(got[n]), _bits(want[n])), (wl.name, n)
        ref = bwd_seq(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.as_f64("g"),
                      inp.as_f64("beta"), inp.as_f64("h0"), inp.cu_seqlens,
                      og.as_f64("dout"), og.as_f64("dhT"))
        errs = {n: _rel(host_f64(got[n]), ref[n]) for n in NAMES}
        print(wl.name, " ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
        assert all(e <= TOL[wl.dtype] for e in errs.values()), (wl.name, errs)
