#!/usr/bin/env python3
"""Benchmark of the gated-delta-rule forward kernel on one MI355X.

One "step" is one gdn_fwd call over one batch of the wide-head workload
(B=4, H=16, T=4096, dk=dv=128, bf16 q/k/v/out, fp32 g/beta, fp32 state with
h0 ~ N(0, 0.02), chunk 64), inputs already resident in HBM.  Four complete
input/output sets (about 1.1 GB) are rotated so that the 256 MB last-level
cache cannot serve a step from the previous one.

Prints ONE JSON line: tokens/s over the timed steps, the roofline of the
kernel (algorithmic HBM bytes per launch / mean launch time measured with
HIP events on the launch stream, against the 8 TB/s HBM3E peak), and the
FP64 oracle timed on the host cores on the same workload.

``--workload decode`` (one token per sequence, B=128 H=16 d=128, nonzero
state) times the token-by-token entry point gdn_fwd_recurrent instead;
``--form`` picks the entry point for any workload; ``--form scan`` times
gdn_fwd_scan (segments with exact entry states from the chunk-map scan:
three launches per step, timed together).

``--pass bwd`` times the backward entry point gdn_bwd on the same workload
(dq, dk, dv, dg, dbeta, dh0 from seeded output gradients dout ~ N(0,1),
dhT ~ N(0,1)); its roofline is the matrix cores' bf16 rate for bf16 storage
with dk = dv = 128 (three full-width kernels, 64-token chunks) and fp32
arithmetic otherwise (four fp32 kernels, 32-token chunks).  ``--pass train``
times a training step for those full-width shapes: gdn_fwd_train (outputs
plus the backward's per-chunk records) followed by gdn_bwd_saved, the
forward's and the backward's products counted together.

``--workload hymo`` / ``hymo_decode`` time the diagonal-decay additive
recurrence with its epilogue (gdn_diag_fwd / gdn_diag_fwd_recurrent) on the
HyMo layer's shape (B=4, T=4096, H=40, S=D=32, bf16) and on one decoding
step of it at batch 256; their lines carry their own metric name.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "gated-delta-rule fwd tokens/s + achieved HBM GB/s (% roofline), 1 MI355X"
CSRC = os.path.join(ROOT, "gated_deltanet_recurrence_delta_amd", "csrc")
# the sources of the kernel each workload's traffic counters were taken on
KERNEL_SRCS = {
    "wide_head": [os.path.join(CSRC, f) for f in ("gdn_fwd_full.hip", "gdn_device.h", "gdn_full_common.h",
                                                  "gdn_launch.h")],
    "hymo": [os.path.join(CSRC, "gdn_diag.hip")],
}
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
COPY_BYTES = 256 << 20  # bytes read (and written) by one calibration copy
METRIC_BWD = "gated-delta-rule bwd tokens/s + achieved fp32 TFLOP/s (% roofline), 1 MI355X"
METRIC_TRAIN = "gated-delta-rule training step (fwd + bwd) tokens/s + achieved bf16 TFLOP/s (% roofline), 1 MI355X"
FP32_PEAK_TFLOPS = 157.3
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores (no sparsity)
METRIC_DIAG = ("diagonal-decay recurrence (HyMo GDN layer) fwd tokens/s + achieved HBM GB/s "
               "(% roofline), 1 MI355X")


def _dev(x):
    """A stored synthetic array (float32, or uint16 bfloat16 bits) as a device tensor."""
    import torch

    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _device_inputs(inp: synth.Inputs):
    return {n: _dev(getattr(inp, n)) for n in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")}


def _host_f64(t):
    import torch

    return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy().astype(np.float64)


def algorithmic_bytes(wl: synth.Workload, has_h0: bool) -> int:
    """Minimum HBM traffic of one call: read q, k, v, g, beta once, write out
    once, read h0 (if given) and write hT once."""
    s = 2 if wl.dtype == "bf16" else 4
    per_token_head = (2 * wl.dk + 2 * wl.dv) * s + 2 * 4
    state = wl.B * wl.H * wl.dk * wl.dv * 4
    return wl.tokens * wl.H * per_token_head + state * (2 if has_h0 else 1)


def kernel_source_hash(workload: str = "wide_head") -> str:
    """sha256[:16] of the code of the kernel sources behind ``workload``:
    comments and whitespace are dropped first, so that editing a comment does
    not disown counter runs taken on the same code."""
    import re

    text = ""
    for path in KERNEL_SRCS[workload]:
        with open(path) as f:
            text += f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = "".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs
    (profiles/traffic_<workload>.json), if they were taken on the current
    kernel source; else None."""
    if workload not in KERNEL_SRCS:
        return None
    try:
        with open(os.path.join(TRAFFIC_DIR, f"traffic_{workload}.json")) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_sha256_16") != kernel_source_hash(workload):
        return None
    return d.get("bytes_per_launch")


def copy_calibration():
    """Three plain device-to-device copies of COPY_BYTES each, before the
    warm-up: under rocprofv3 --pmc their FETCH_SIZE / WRITE_SIZE readings
    give the bytes per counted KiB."""
    import torch

    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def copy_reference(nbytes: int, stream) -> float:
    """Achievable-bandwidth reference: GB/s of a plain device-to-device copy
    moving ``nbytes`` (half read, half written) per call, over four rotated
    buffer pairs so that the last-level cache cannot serve it."""
    import torch

    n = max(1, nbytes // 8)  # float32 elements per buffer
    src = [torch.empty(n, dtype=torch.float32, device="cuda").uniform_() for _ in range(4)]
    dst = [torch.empty_like(src[0]) for _ in range(4)]
    with torch.cuda.stream(stream):
        for i in range(20):
            dst[i % 4].copy_(src[i % 4])
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(40)]
        for i, (a, b) in enumerate(ev):
            a.record(stream)
            dst[i % 4].copy_(src[i % 4])
            b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    med_s = t[len(t) // 2] / 1e3
    del src, dst
    return 2 * n * 4 / med_s / 1e9


def timing_record(launch_ms, settle_launches: int, cold_us: float) -> dict:
    """How the timed launches were taken: the untimed settling launches that
    preceded them, the first call of the process, and whether the clock had
    settled -- the mean of the first quarter of the timed launches within 3%
    of the mean of the last quarter."""
    q = max(1, len(launch_ms) // 4)
    first, last = float(np.mean(launch_ms[:q])), float(np.mean(launch_ms[-q:]))
    return {"settle_launches": settle_launches, "cold_first_call_us": cold_us,
            "first_quarter_mean_us": first * 1e3, "last_quarter_mean_us": last * 1e3,
            "clock_settled": bool(abs(first - last) <= 0.03 * last)}


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def chain_errors(inp: synth.Inputs, o, hT, o_ref, h_ref):
    """Worst per-chain infinity-norm relative error of out and hT, each
    chain on its own scale, with that chain's (sequence, head)."""
    def ratio(num, den):
        return np.where(num > 0, num / np.where(den > 0, den, 1.0) + np.where(den > 0, 0, np.inf), 0.0)

    eh = ratio(np.abs(hT - h_ref).max(axis=(2, 3)), np.abs(h_ref).max(axis=(2, 3)))
    if inp.cu_seqlens is None:
        eo = ratio(np.abs(o - o_ref).max(axis=(1, 3)), np.abs(o_ref).max(axis=(1, 3)))
    else:
        eo = np.zeros_like(eh)
        cu = inp.cu_seqlens
        for n in range(len(cu) - 1):
            a, b = int(cu[n]), int(cu[n + 1])
            if b > a:
                eo[n] = ratio(np.abs(o[a:b] - o_ref[a:b]).max(axis=(0, 2)),
                              np.abs(o_ref[a:b]).max(axis=(0, 2)))
    worst = np.maximum(eo, eh)
    b, h = np.unravel_index(int(np.argmax(worst)), worst.shape)
    return float(eo.max()), float(eh.max()), (int(b), int(h))


def cpu_baseline(inp: synth.Inputs, out=None, hT=None, check=True):
    """The FP64 oracle on the host cores over the whole workload (timed).
    When the GPU's (out, hT) are given, the same oracle results also check
    them (infinity-norm relative error per tensor, within the dtype's
    tolerance) before any number is reported.  Returns (record, errs)."""
    import oracle

    a = [inp.as_f64(n) for n in ("q", "k", "v", "g", "beta", "h0")]
    cores = os.cpu_count() or 1
    oracle.build(force=False)
    t0 = time.perf_counter()
    o_ref, h_ref = oracle.fwd_seq(*a, cu_seqlens=inp.cu_seqlens, nthreads=cores)
    dt = time.perf_counter() - t0
    wl = inp.wl
    nchains = (len(inp.cu_seqlens) - 1 if inp.cu_seqlens is not None else wl.B) * wl.H
    rec = {"value": wl.tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"whole workload ({nchains} chains, {wl.tokens} tokens x {wl.H} heads), "
                     f"{dt:.2f} s wall on {cores} threads"}
    errs = None
    if check and out is not None:
        o, h = _host_f64(out), _host_f64(hT)
        eo = oracle.rel_err(o, o_ref)
        eh = oracle.rel_err(h, h_ref)
        co, ch, worst = chain_errors(inp, o, h, o_ref, h_ref)
        tol = 2e-2 if wl.dtype == "bf16" else 1e-4
        if not max(eo, eh, co, ch) <= tol:
            raise SystemExit(f"parity check failed: rel err out {eo:.3e} hT {eh:.3e}, worst chain "
                             f"{worst} out {co:.3e} hT {ch:.3e} > {tol}")
        errs = {"rel_err_out": eo, "rel_err_hT": eh, "worst_chain": list(worst),
                "worst_chain_rel_err_out": co, "worst_chain_rel_err_hT": ch}
    return rec, errs


def diag_algorithmic_bytes(wl, has_h0: bool, has_gate: bool) -> int:
    """Minimum HBM traffic of one diagonal-decay call: read v, b, c, g (and
    gate) once, write out once, read h0 (if given), write hT, read A_log/D."""
    s = 2 if wl.dtype == "bf16" else 4
    per_token_head = (2 * wl.D + 2 * wl.S) * s + 4 + (4 if has_gate else 0)
    state = wl.B * wl.H * wl.S * wl.D * 4
    params = wl.H * wl.S * 4 + wl.H * 4
    return wl.tokens * wl.H * per_token_head + state * (2 if has_h0 else 1) + params


def diag_main(args):
    """The diagonal-decay form: same protocol as ``main`` (rotated sets, HIP
    events on the launch stream, CPU oracle leg that also checks parity)."""
    import torch

    import gated_deltanet_recurrence_delta_amd as gdn
    import synth.diag as sd

    wl = sd.WORKLOADS[args.workload]
    form = args.form or ("recurrent" if wl.T == 1 else "chunked")
    inp = sd.generate(wl)

    names = ("v", "b", "c", "g", "A_log", "Dskip", "gate", "h0", "cu_seqlens")
    sets = []
    for _ in range(max(1, args.sets)):
        d = {n: _dev(getattr(inp, n)) for n in names}
        d["out"] = torch.empty(d["v"].shape, dtype=d["v"].dtype, device="cuda")
        d["hT"] = torch.empty((wl.B, wl.H, wl.S, wl.D), dtype=torch.float32, device="cuda")
        sets.append(d)
    stream = torch.cuda.current_stream()
    f = gdn.diag_fwd if form == "chunked" else gdn.diag_fwd_recurrent
    for d in sets:
        f(d["v"], d["b"], d["c"], d["g"], d["A_log"], D=d["Dskip"], gate=d["gate"], h0=d["h0"],
          cu_seqlens=d["cu_seqlens"], out=d["out"], hT=d["hT"], stream=stream)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    calls = [tuple(ptr(d[n]) for n in names + ("out", "hT")) for d in sets]
    dtype_code = gdn.GDN_BF16 if wl.dtype == "bf16" else gdn.GDN_F32
    sh = stream.cuda_stream
    if form == "chunked":
        raw = gdn.load().gdn_diag_fwd
        tail = (wl.B, wl.T, wl.H, wl.S, wl.D, sh, dtype_code, 0)
    else:
        raw = gdn.load().gdn_diag_fwd_recurrent
        tail = (wl.B, wl.T, wl.H, wl.S, wl.D, sh, dtype_code)

    def step(i):
        rc = raw(*calls[i % len(calls)], *tail)
        if rc != 0:
            raise SystemExit(f"diagonal-decay {form} entry point failed with status {rc}")

    alg = diag_algorithmic_bytes(wl, inp.h0 is not None, inp.gate is not None)
    if args.copy_calibration:
        copy_calibration()
    copy_gbs = copy_reference(alg, stream)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = np.array([a.elapsed_time(e) for a, e in zip(starts, ends)])
    ms_per_step = wall * 1e3 / args.steps
    mean_launch_s = float(launch_ms.mean()) / 1e3
    achieved = alg / mean_launch_s / 1e9
    rec = {
        "metric": METRIC_DIAG,
        "value": wl.tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; v N(0,1), b,c N(0,1/S), g=sigmoid(N(0,1)), "
                "A_log=log(h+1)+N(0,0.25^2), D=1+N(0,0.1^2), gate=sigmoid(N(0,0.25^2)))",
        "config": {"workload": f"{wl.name}: B={wl.B} H={wl.H} T={wl.T} S={wl.S} D={wl.D} "
                               f"{wl.dtype} " + ("chunk=64" if form == "chunked" else "token-by-token")
                               + " epilogue D*v, gate",
                   "entry_point": "gdn_diag_fwd" if form == "chunked" else "gdn_diag_fwd_recurrent",
                   "tokens_per_step": wl.tokens, "rotated_sets": len(sets)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(args.workload) if form == "chunked" else None,
                     "copy_GBs": copy_gbs, "frac_of_copy": achieved / copy_gbs,
                     "algorithmic_bytes": alg, "mean_launch_us": mean_launch_s * 1e6,
                     "p10_us": float(np.percentile(launch_ms, 10)) * 1e3,
                     "p50_us": float(np.percentile(launch_ms, 50)) * 1e3,
                     "p90_us": float(np.percentile(launch_ms, 90)) * 1e3},
    }
    if not args.no_cpu:
        from oracle import diag as odiag
        from oracle import rel_err

        t0 = time.perf_counter()
        a = {n: None if getattr(inp, n) is None else inp.as_f64(n) for n in names[:-1]}
        o_ref, h_ref = odiag.diag_fwd_seq(a["v"], a["b"], a["c"], a["g"], a["A_log"], a["h0"],
                                          None, a["Dskip"], a["gate"])
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": wl.tokens / dt, "unit": "tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"whole workload ({wl.B * wl.H} chains x {wl.T} tokens), "
                                         f"NumPy token loop, {dt:.2f} s wall"}
        if not args.no_parity:
            # the same oracle results check sets[0]'s outputs (from its last
            # timed step: identical inputs, deterministic kernel)
            eo = rel_err(sets[0]["out"].float().cpu().numpy(), o_ref)
            eh = rel_err(sets[0]["hT"].cpu().numpy(), h_ref)
            if not (eo <= 2e-2 and eh <= 2e-2):
                raise SystemExit(f"parity check failed: rel err out {eo:.3e} hT {eh:.3e}")
            rec["parity"] = {"rel_err_out": eo, "rel_err_hT": eh,
                             "chains": "all (the oracle leg's whole-workload run)"}
    print(json.dumps(rec), flush=True)


def bwd_full_width(wl: synth.Workload) -> bool:
    """gdn_bwd runs the full-width bf16 kernels (64-token chunks) for these shapes."""
    return wl.dtype == "bf16" and wl.dk == 128 and wl.dv == 128


def bwd_flops_full(wl: synth.Workload, lens) -> int:
    """Floating-point operations of one full-width gdn_bwd call (bf16, dk = dv
    = d = 128, C = 64-token chunks; 2 per multiply-add; products with a
    triangular factor counted at half).  Per chunk and head:
      states   K K^T (C^2 d / 2), the triangular inverse (C^3 / 6), K M and
               K^T diag(w) U (2 C d^2), T diag(beta) X (C^2 d / 2)
      adjoint  K K^T and Q K^T (C^2 d), the inverse (C^3 / 6), K dM',
               Q^T (Gam dO), K^T W (3 C d^2), P^T dO and T^T dU (C^2 d)
      grad     K K^T, Q K^T, dX U^T, dO U^T (2 C^2 d), dO M^T, dX M^T,
               U dM'^T (3 C d^2), (dP.E) K, G K, G^T K, (dP.E)^T Q (2 C^2 d)."""
    C, d = 64, wl.dk
    per_chunk = (C * C * d // 2 + C ** 3 // 6 + 2 * C * d * d + C * C * d // 2
                 + C * C * d + C ** 3 // 6 + 3 * C * d * d + C * C * d
                 + 2 * C * C * d + 3 * C * d * d + 2 * C * C * d)
    chunks = sum((int(n) + C - 1) // C for n in lens)
    return 2 * per_chunk * chunks * wl.H


def fwd_flops_full(wl: synth.Workload, lens) -> int:
    """Floating-point operations of the full-width forward (64-token chunks):
    per chunk and head 3 C d^2 multiply-adds (K M, Q M and the state update
    K^T W), 2 C^2 d (K K^T, Q K^T, T X and P U, each triangular, at half) and
    C^3 / 6 (one triangular inverse); a partial chunk counts as a whole one."""
    C, d = 64, wl.dk
    per = 3 * C * d * wl.dv + 2 * C * C * d + C ** 3 // 6
    return 2 * per * sum((int(n) + C - 1) // C for n in lens) * wl.H


def bwd_flops(wl: synth.Workload, lens) -> int:
    """Floating-point operations of one gdn_bwd call as its four kernels
    compute it (32-token chunks; 2 per multiply-add).  Per chunk of L <= 32
    tokens (C = 32, the padded chunk), per head:
      prep     K K^T and Q K^T (2 C^2 dk), the triangular inverse (C^3 / 6)
      states   K M, K^T diag(w) U (2 C dk dv), T X (C^2 dv / 2)
      adjoint  K dM', Q^T dO, K^T dX (3 C dk dv), P^T dO, T^T dU (C^2 dv)
      grad     K M, Q M, K dM', dO M^T, dX M^T, U dM'^T (6 C dk dv),
               T X, P^T dO, T^T dU (3 C^2 dv / 2), dX U^T, dO U^T (2 C^2 dv),
               K K^T (C^2 dk / 2), (dP.E) K, G K, G^T K, (dP.E)^T Q (4 C^2 dk)."""
    C, dk, dv = 32, wl.dk, wl.dv
    per_chunk = (2 * C * C * dk + C ** 3 // 6
                 + 2 * C * dk * dv + C * C * dv // 2
                 + 3 * C * dk * dv + C * C * dv
                 + 6 * C * dk * dv + 3 * C * C * dv // 2 + 2 * C * C * dv
                 + C * C * dk // 2 + 4 * C * C * dk)
    chunks = sum((int(n) + C - 1) // C for n in lens)
    return 2 * per_chunk * chunks * wl.H


def bwd_main(args):
    """The backward pass: same protocol as ``main`` (rotated sets, HIP events
    on the launch stream around each gdn_bwd call, a CPU oracle leg on two
    chains whose results also check those chains).  ``--pass train`` times a
    training step instead: gdn_fwd_train (outputs and the backward's
    records) then gdn_bwd_saved, bf16 with dk = dv = 128 only."""
    import torch

    import gated_deltanet_recurrence_delta_amd as gdn

    wl = synth.WORKLOADS[args.workload]
    train = args.direction == "train"
    if train and not bwd_full_width(wl):
        raise SystemExit("--pass train needs bf16 storage with dk = dv = 128")
    inp = synth.generate(wl)
    og = synth.output_grads(inp, 1000 + wl.seed)
    B = len(inp.cu_seqlens) - 1 if inp.cu_seqlens is not None else wl.B
    T = int(inp.cu_seqlens[-1]) if inp.cu_seqlens is not None else wl.T
    lens = (np.diff(inp.cu_seqlens) if inp.cu_seqlens is not None else [wl.T] * wl.B)
    need = gdn.gdn_bwd_workspace_size(B, T, wl.H, wl.dk, wl.dv, inp.cu_seqlens is not None)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    sets = []
    for _ in range(max(1, args.sets)):
        d = _device_inputs(inp)
        d["dout"], d["dhT"] = _dev(og.dout), _dev(og.dhT)
        for n, like in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg", "g"), ("dbeta", "beta")):
            d[n] = torch.empty_like(d[like])
        d["dh0"] = torch.empty((B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
        d["out"] = torch.empty_like(d["v"])
        d["hT"] = torch.empty((B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
        sets.append(d)
    stream = torch.cuda.current_stream()
    d0 = sets[0]
    if train:
        gdn.fwd_train(d0["q"], d0["k"], d0["v"], d0["g"], d0["beta"], d0["h0"], d0["cu_seqlens"],
                      out=d0["out"], hT=d0["hT"], workspace=ws, stream=stream)
    first = gdn.bwd(d0["q"], d0["k"], d0["v"], d0["g"], d0["beta"], d0["dout"], h0=d0["h0"],
                    cu_seqlens=d0["cu_seqlens"], dhT=d0["dhT"], workspace=ws, stream=stream,
                    saved=train)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    names = ("q", "k", "v", "g", "beta", "h0", "cu_seqlens", "dout", "dhT", "dq", "dk", "dv",
             "dg", "dbeta", "dh0")
    calls = [tuple(ptr(d[n]) for n in names) for d in sets]
    dtype_code = gdn.GDN_BF16 if wl.dtype == "bf16" else gdn.GDN_F32
    raw = gdn.load().gdn_bwd_saved if train else gdn.load().gdn_bwd
    tail = (ws.data_ptr(), need, B, T, wl.H, wl.dk, wl.dv, stream.cuda_stream, dtype_code)
    fnames = ("q", "k", "v", "g", "beta", "h0", "cu_seqlens", "out", "hT")
    fcalls = [tuple(ptr(d[n]) for n in fnames) for d in sets]
    raw_fwd = gdn.load().gdn_fwd_train
    ftail = (B, T, wl.H, wl.dk, wl.dv, stream.cuda_stream, dtype_code, 0, ws.data_ptr(), need)

    def step(i):
        if train:
            rc = raw_fwd(*fcalls[i % len(fcalls)], *ftail)
            if rc != 0:
                raise SystemExit(f"gdn_fwd_train failed with status {rc}")
        rc = raw(*calls[i % len(calls)], *tail)
        if rc != 0:
            raise SystemExit(f"gdn_bwd failed with status {rc}")

    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = np.array([a.elapsed_time(e) for a, e in zip(starts, ends)])
    ms_per_step = wall * 1e3 / args.steps
    mean_s = float(launch_ms.mean()) / 1e3
    full = bwd_full_width(wl)
    flops = bwd_flops_full(wl, lens) if full else bwd_flops(wl, lens)
    if train:
        flops += fwd_flops_full(wl, lens)
    peak = BF16_PEAK_TFLOPS if full else FP32_PEAK_TFLOPS
    achieved = flops / mean_s / 1e12
    rec = {
        "metric": METRIC_TRAIN if train else METRIC_BWD,
        "value": wl.tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), beta=sigmoid(N(0,1)), "
                "g=-softplus(N(%g,1)), dout N(0,1), dhT N(0,1))" % wl.g_mean,
        "config": {"workload": f"{wl.name}: B={wl.B} H={wl.H} T={wl.T} dk={wl.dk} dv={wl.dv} "
                               f"{wl.dtype} " + ("training step (forward with records, backward from them), "
                                                 if train else "backward, ")
                               + ("64-token chunks" if full else "32-token chunks")
                               + (" varlen" if wl.varlen else ""),
                   "entry_point": "gdn_fwd_train + gdn_bwd_saved" if train else "gdn_bwd",
                   "tokens_per_step": wl.tokens,
                   "rotated_sets": len(sets), "workspace_bytes": need},
        "roofline": {"bound": "mfma" if full else "alu", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": None,
                     "kernel": ("gdn_fwd_train and gdn_bwd_saved, their three kernels (forward with records, "
                                "adjoint, grad) of one step, bf16 matrix cores" if train else
                                "gdn_bwd, its three kernels (states, adjoint, grad) of one call, "
                                "bf16 matrix cores" if full else "gdn_bwd, all four kernels of one call"),
                     "algorithmic_flops": flops, "mean_launch_us": mean_s * 1e6,
                     "p10_us": float(np.percentile(launch_ms, 10)) * 1e3,
                     "p50_us": float(np.percentile(launch_ms, 50)) * 1e3,
                     "p90_us": float(np.percentile(launch_ms, 90)) * 1e3},
    }
    if not args.no_cpu and inp.cu_seqlens is None:
        from oracle.bwd import bwd_seq

        # the oracle on two chains, (first sequence, first head) and (last,
        # last); its results also check those chains of the first call
        chains = sorted({(0, 0), (wl.B - 1, wl.H - 1)})
        refs = {}
        t0 = time.perf_counter()
        for b, h in chains:
            cut = lambda x: None if x is None else x[b:b + 1, :, h:h + 1]
            refs[(b, h)] = bwd_seq(
                *(cut(inp.as_f64(n)) for n in ("q", "k", "v", "g", "beta")),
                None if inp.h0 is None else inp.as_f64("h0")[b:b + 1, h:h + 1], None,
                cut(og.as_f64("dout")),
                None if og.dhT is None else og.as_f64("dhT")[b:b + 1, h:h + 1])
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": (len(chains) * wl.T / wl.H) / dt, "unit": "tokens/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{len(chains)} chains of {wl.T} tokens (first sequence "
                                         f"first head, last sequence last head), NumPy reverse "
                                         f"sweep, {dt:.2f} s wall; one chain is 1/{wl.H} of a "
                                         "token's heads"}
        if not args.no_parity:
            worst = {}
            for (b, h), ref in refs.items():
                for n in ("dq", "dk", "dv", "dg", "dbeta"):
                    got = _host_f64(first[n][b:b + 1, :, h:h + 1])
                    e = float(np.max(np.abs(got - ref[n])) / max(np.max(np.abs(ref[n])), 1e-30))
                    worst[n] = max(worst.get(n, 0.0), e)
                got = _host_f64(first["dh0"][b:b + 1, h:h + 1])
                e = float(np.max(np.abs(got - ref["dh0"])) / max(np.max(np.abs(ref["dh0"])), 1e-30))
                worst["dh0"] = max(worst.get("dh0", 0.0), e)
            tol = 2e-2 if wl.dtype == "bf16" else 1e-4
            if not all(e <= tol for e in worst.values()):
                raise SystemExit(f"parity check failed: {worst}")
            rec["parity"] = dict(worst, chains="(first sequence, first head), (last, last)")
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # about 40 ms of warm-up: the first ~10 ms of launches after an idle
    # period run at a lower GPU clock
    ap.add_argument("--warmup", type=int, default=300)
    import synth.diag as sd

    ap.add_argument("--workload", default="wide_head",
                    choices=sorted(synth.WORKLOADS) + sorted(sd.WORKLOADS))
    ap.add_argument("--form", choices=("chunked", "recurrent", "scan"), default=None,
                    help="entry point (default: recurrent for the decode workload, "
                         "chunked otherwise)")
    ap.add_argument("--pass", dest="direction", choices=("fwd", "bwd", "train"), default="fwd",
                    help="forward (default) or backward entry point")
    ap.add_argument("--sets", type=int, default=4, help="rotated input/output sets")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the parity check made with the oracle leg's results")
    ap.add_argument("--no-segments", action="store_true",
                    help="pass GDN_FLAG_NO_SEGMENTS: every chain runs from its start")
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="untimed launches for at least this long before the warm-up steps, "
                         "so that the timed steps run at the clock the GPU settles to under load")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run three plain 256 MiB device-to-device copies, whose HBM "
                         "counter readings calibrate the kernel's FETCH_SIZE/WRITE_SIZE")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); chains shard across GPUs with no communication, "
              "so there is no multi-GPU step to time.", file=sys.stderr)
        sys.exit(2)

    if args.workload in sd.WORKLOADS:
        if args.direction != "fwd":
            raise SystemExit("the diagonal-decay form has no backward entry point")
        return diag_main(args)
    if args.direction in ("bwd", "train"):
        return bwd_main(args)

    import torch

    import gated_deltanet_recurrence_delta_amd as gdn

    wl = synth.WORKLOADS[args.workload]
    form = args.form or ("recurrent" if args.workload == "decode" else "chunked")
    inp = synth.generate(wl)
    sets = []
    for _ in range(max(1, args.sets)):
        d = _device_inputs(inp)
        d["out"] = torch.empty(d["v"].shape, dtype=d["v"].dtype, device="cuda")
        d["hT"] = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
        sets.append(d)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ws = None
    if form == "scan":
        # one workspace for every set: the calls are serialised on the stream
        need = gdn.gdn_fwd_scan_workspace_size(
            len(inp.cu_seqlens) - 1 if inp.cu_seqlens is not None else wl.B,
            int(inp.cu_seqlens[-1]) if inp.cu_seqlens is not None else wl.T, wl.H, wl.dk, wl.dv,
            inp.cu_seqlens is not None, gdn.GDN_BF16 if wl.dtype == "bf16" else gdn.GDN_F32, wl.chunk)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    # Validate once through the checked wrapper, then time the raw C entry
    # point with pre-extracted pointers so host overhead stays off the clock.
    # The first call of the process is also timed on its own: it includes
    # loading the kernel's code object and a GPU that has been idle.
    cold = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for i, d in enumerate(sets):
        if i == 0:
            cold[0].record(stream)
        if form == "recurrent":
            gdn.fwd_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                              out=d["out"], hT=d["hT"], stream=stream)
        elif form == "scan":
            gdn.fwd_scan(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                         chunk=wl.chunk, out=d["out"], hT=d["hT"], stream=stream, workspace=ws)
        else:
            gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                    chunk=wl.chunk, out=d["out"], hT=d["hT"], stream=stream,
                    segments=not args.no_segments)
        if i == 0:
            cold[1].record(stream)
    torch.cuda.synchronize()
    cold_us = cold[0].elapsed_time(cold[1]) * 1e3
    ptr = lambda t: 0 if t is None else t.data_ptr()
    dtype_code = gdn.GDN_BF16 if wl.dtype == "bf16" else gdn.GDN_F32
    B = len(inp.cu_seqlens) - 1 if inp.cu_seqlens is not None else wl.B
    T = int(inp.cu_seqlens[-1]) if inp.cu_seqlens is not None else wl.T
    calls = [tuple(ptr(d[n]) for n in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens", "out", "hT"))
             for d in sets]
    sh = stream.cuda_stream
    if form == "recurrent":
        raw = gdn.load().gdn_fwd_recurrent
        tail = (B, T, wl.H, wl.dk, wl.dv, sh, dtype_code)
    elif form == "scan":
        raw = gdn.load().gdn_fwd_scan
        tail = (B, T, wl.H, wl.dk, wl.dv, sh, dtype_code, wl.chunk, ws.data_ptr(), ws.numel())
    else:
        raw = gdn.load().gdn_fwd
        flags = gdn.GDN_FLAG_NO_SEGMENTS if args.no_segments else 0
        tail = (B, T, wl.H, wl.dk, wl.dv, sh, dtype_code, wl.chunk, flags)

    def step(i):
        rc = raw(*calls[i % len(calls)], *tail)
        if rc != 0:
            raise SystemExit(f"{form} entry point failed with status {rc}")

    if args.copy_calibration:
        copy_calibration()

    copy_gbs = copy_reference(algorithmic_bytes(wl, inp.h0 is not None), stream)

    # Untimed launches for at least --settle-ms, then the warm-up steps,
    # which lead straight into the timed ones so that the GPU is not left
    # idle (and its clock low) between them; the oracle leg (timing and
    # parity) runs after the timed steps.
    torch.cuda.synchronize()
    settle_n = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(16):
            step(settle_n)
            settle_n += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])

    ms_per_step = wall * 1e3 / args.steps
    tokens = wl.tokens
    alg = algorithmic_bytes(wl, inp.h0 is not None)
    mean_launch_s = float(launch_ms.mean()) / 1e3
    achieved = alg / mean_launch_s / 1e9
    traffic = measured_traffic(args.workload) if form == "chunked" else None

    rec = {
        "metric": METRIC,
        "value": tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), "
                "beta=sigmoid(N(0,1)), " + ("g=0)" if wl.no_decay else "g=-softplus(N(%g,1)))" % wl.g_mean),
        "config": {"workload": f"{wl.name}: B={wl.B} H={wl.H} T={wl.T} dk={wl.dk} dv={wl.dv} "
                               f"{wl.dtype} " + ("token-by-token" if form == "recurrent"
                                                 else f"chunk={wl.chunk}")
                               + (" varlen" if wl.varlen else ""),
                   "entry_point": {"chunked": "gdn_fwd", "recurrent": "gdn_fwd_recurrent",
                                   "scan": "gdn_fwd_scan"}[form],
                   "tokens_per_step": tokens, "rotated_sets": len(sets)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "copy_GBs": copy_gbs, "frac_of_copy": achieved / copy_gbs,
                     "algorithmic_bytes": alg, "mean_launch_us": mean_launch_s * 1e6,
                     "p10_us": float(np.percentile(launch_ms, 10)) * 1e3,
                     "p50_us": float(np.percentile(launch_ms, 50)) * 1e3,
                     "p90_us": float(np.percentile(launch_ms, 90)) * 1e3},
        "timing": timing_record(launch_ms, settle_n, cold_us),
    }
    if not args.no_cpu:
        # sets[0]'s outputs come from its last timed step (identical inputs,
        # bitwise-deterministic kernel)
        rec["cpu_baseline"], errs = cpu_baseline(inp, sets[0]["out"], sets[0]["hT"],
                                                 check=not args.no_parity)
        if errs is not None:
            rec["parity"] = dict(errs, chains="all (the oracle leg's whole-workload run), each "
                                              "also on its own scale")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
