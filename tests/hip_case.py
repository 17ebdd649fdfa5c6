"""Shared helpers for the GPU tests: move synthetic inputs to the device,
call the HIP path through the C ABI, and evaluate the FP64 oracle on the
same stored values."""
from __future__ import annotations

import numpy as np

import oracle
import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}


def dev(x):
    import torch

    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host_f64(t):
    import torch

    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def device_inputs(inp: synth.Inputs):
    return dict(q=dev(inp.q), k=dev(inp.k), v=dev(inp.v), g=dev(inp.g), beta=dev(inp.beta),
                h0=dev(inp.h0), cu_seqlens=dev(inp.cu_seqlens))


def run_hip(inp: synth.Inputs, chunk=None, d=None, **kw):
    """(out, hT) as torch device tensors."""
    import torch

    import gated_deltanet_recurrence_delta_amd as gdn

    d = d or device_inputs(inp)
    out, hT = gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                      chunk=chunk if chunk is not None else inp.wl.chunk, **kw)
    torch.cuda.synchronize()
    return out, hT


def run_hip_recurrent(inp: synth.Inputs, d=None, **kw):
    """(out, hT) of the token-by-token entry point as torch device tensors."""
    import torch
    import gated_deltanet_recurrence_delta_amd as gdn

    d = d or device_inputs(inp)
    out, hT = gdn.fwd_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                                d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return out, hT


def run_oracle(inp: synth.Inputs, chains=None):
    a = [inp.as_f64(n) for n in ("q", "k", "v", "g", "beta", "h0")]
    return oracle.fwd_seq(*a, cu_seqlens=inp.cu_seqlens, chains=chains)


def chain_slices(inp: synth.Inputs, c: int):
    """(index of chain c's outputs in out, index of its state in hT)."""
    H = inp.wl.H
    b, h = divmod(c, H)
    if inp.cu_seqlens is not None:
        s, e = synth.chain_bounds(inp, b)
        return (slice(s, e), h), (b, h)
    return (b, slice(None), h), (b, h)


def compare(inp: synth.Inputs, out_hip, hT_hip, chains=None):
    """Max relative errors (out, hT) of the HIP result against the oracle,
    over all chains or over the listed chain ids."""
    o_ref, h_ref = run_oracle(inp, chains)
    o = host_f64(out_hip)
    hT = host_f64(hT_hip)
    if chains is None:
        return oracle.rel_err(o, o_ref), oracle.rel_err(hT, h_ref)
    # Infinity-norm relative error over the sampled part of each tensor.
    num_o = den_o = num_h = den_h = 0.0
    for c in chains:
        so, sh = chain_slices(inp, c)
        if o_ref[so].size:
            num_o = max(num_o, float(np.max(np.abs(o[so] - o_ref[so]))))
            den_o = max(den_o, float(np.max(np.abs(o_ref[so]))))
        num_h = max(num_h, float(np.max(np.abs(hT[sh] - h_ref[sh]))))
        den_h = max(den_h, float(np.max(np.abs(h_ref[sh]))))
    ratio = lambda n, d: 0.0 if n == 0.0 else (n / d if d > 0 else float("inf"))
    return ratio(num_o, den_o), ratio(num_h, den_h)
