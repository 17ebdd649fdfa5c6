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


def run_hip_scan(inp: synth.Inputs, d=None, **kw):
    """(out, hT) of the chunk-map scan entry point as torch device tensors."""
    import torch

    import gated_deltanet_recurrence_delta_amd as gdn

    d = d or device_inputs(inp)
    out, hT = gdn.fwd_scan(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                           chunk=inp.wl.chunk, **kw)
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


def _ratio(num, den):
    """max|err| / max|ref| with 0/0 -> 0 (elementwise over arrays)."""
    num = np.asarray(num, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    out = np.zeros(np.broadcast(num, den).shape)
    nz = num > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        out[nz] = np.where(den[nz] > 0, num[nz] / np.where(den[nz] > 0, den[nz], 1.0), np.inf)
    return out


def per_chain_errors(inp: synth.Inputs, o, hT, o_ref, h_ref):
    """Infinity-norm relative error of every chain on its own scale:
    (e_out[B, H], e_hT[B, H]) with e = max|x - ref| / max|ref| over the
    chain's slice of out (its tokens, its head) and of hT."""
    B = hT.shape[0]
    H = hT.shape[1]
    dh = np.abs(hT - h_ref).max(axis=(2, 3))
    rh = np.abs(h_ref).max(axis=(2, 3))
    e_h = _ratio(dh, rh)
    if inp.cu_seqlens is None:
        if o.size:
            do = np.abs(o - o_ref).max(axis=(1, 3))
            ro = np.abs(o_ref).max(axis=(1, 3))
            e_o = _ratio(do, ro)
        else:
            e_o = np.zeros((B, H))
    else:
        e_o = np.zeros((B, H))
        for n in range(B):
            s, e = synth.chain_bounds(inp, n)
            if e > s:
                e_o[n] = _ratio(np.abs(o[s:e] - o_ref[s:e]).max(axis=(0, 2)),
                                np.abs(o_ref[s:e]).max(axis=(0, 2)))
    return e_o, e_h


def compare_all(inp: synth.Inputs, out_hip, hT_hip):
    """The oracle on every chain; returns a dict with the whole-tensor
    errors (out, hT) and the worst chain's own-scale errors with its
    (sequence, head)."""
    o_ref, h_ref = run_oracle(inp)
    o = host_f64(out_hip)
    hT = host_f64(hT_hip)
    e_o, e_h = per_chain_errors(inp, o, hT, o_ref, h_ref)
    worst = np.maximum(e_o, e_h)
    b, h = np.unravel_index(int(np.argmax(worst)), worst.shape)
    return {"out": oracle.rel_err(o, o_ref), "hT": oracle.rel_err(hT, h_ref),
            "chain_out": float(e_o.max()), "chain_hT": float(e_h.max()),
            "worst_chain": (int(b), int(h))}


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
