"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the algorithmic
byte and flop counts the roofline divides by, and the source hash that
decides whether committed counter readings still describe the kernel."""
import os
import subprocess
import sys

import bench
import numpy as np
import synth
import synth.diag as sd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_without_touching_the_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_wide_head_algorithmic_bytes():
    """262,144 token-heads x (2*128 + 2*128) bf16 elements + 8 bytes of g and
    beta, plus h0 read and hT written (64 chains x 128 x 128 fp32 each)."""
    wl = synth.WORKLOADS["wide_head"]
    per = (2 * 128 + 2 * 128) * 2 + 8
    assert bench.algorithmic_bytes(wl, True) == 4 * 4096 * 16 * per + 2 * 64 * 128 * 128 * 4
    assert bench.algorithmic_bytes(wl, True) == 278_921_216


def test_hymo_algorithmic_bytes():
    wl = sd.WORKLOADS["hymo"]
    b = bench.diag_algorithmic_bytes(wl, False, True)
    assert b == 4 * 4096 * 40 * ((2 * 32 + 2 * 32) * 2 + 8) + 160 * 32 * 32 * 4 + 40 * 32 * 4 + 40 * 4
    assert abs(b / 1e6 - 173.7) < 0.05


def test_backward_flops_count_chunks_per_sequence():
    wl = synth.WORKLOADS["wide_head"]
    f = bench.bwd_flops(wl, [wl.T] * wl.B)
    assert f == 119_274_815_488
    # a ragged sequence counts its partial chunk as a whole chunk
    assert bench.bwd_flops(wl, [33]) == 2 * bench.bwd_flops(wl, [32])


def test_full_width_backward_flops():
    """bf16 with dk = dv = 128 runs the 64-token full-width kernels; per
    chunk and head: 8 C d^2 (dense products), 7 C^2 d (chunk-square ones,
    triangular ones at half) and C^3 / 3 (two triangular inverses)."""
    wl = synth.WORKLOADS["wide_head"]
    assert bench.bwd_full_width(wl) and not bench.bwd_full_width(synth.WORKLOADS["small_state"])
    C, d = 64, 128
    per = 8 * C * d * d + 7 * C * C * d + 2 * (C ** 3 // 6)
    assert bench.bwd_flops_full(wl, [wl.T] * wl.B) == 2 * per * 64 * wl.B * wl.H
    assert bench.bwd_flops_full(wl, [65]) == 2 * bench.bwd_flops_full(wl, [64])


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", {"wide_head": [str(src)]})
    h1 = bench.kernel_source_hash()
    src.write_text("/* a note */\nint f(int x)   {\n\n  return x + 1;  // changed comment\n}\n")
    assert bench.kernel_source_hash() == h1
    src.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_source_hash() != h1


def test_chain_errors_scale_each_chain_on_its_own():
    """A chain whose outputs are 100x smaller than the tensor's largest is
    judged against its own largest value, not the tensor's."""
    inp = synth.generate(synth.custom(name="ce", seed=1, B=2, T=3, H=2, dk=2, dv=2))
    o_ref = np.ones((2, 3, 2, 2))
    o_ref[1, :, 0] = 0.01
    h_ref = np.ones((2, 2, 2, 2))
    o = o_ref.copy()
    o[1, 2, 0, 1] += 0.001  # 0.1 % of the tensor's scale, 10 % of the chain's
    co, ch, worst = bench.chain_errors(inp, o, h_ref.copy(), o_ref, h_ref)
    assert abs(co - 0.1) < 1e-12 and ch == 0.0 and worst == (1, 0)


def test_timing_record_settled_flag():
    flat = np.full(40, 0.1)
    r = bench.timing_record(flat, 5, 123.0)
    assert r["clock_settled"] and r["settle_launches"] == 5 and r["cold_first_call_us"] == 123.0
    ramp = np.concatenate([np.full(10, 0.12), np.full(30, 0.1)])
    assert not bench.timing_record(ramp, 0, 1.0)["clock_settled"]


def test_measured_traffic_follows_each_workloads_sources(tmp_path, monkeypatch):
    """A counter file counts only while its hash matches that workload's
    sources; other workloads and unknown names report None."""
    import json

    srcs = {}
    for w in ("wide_head", "hymo"):
        f = tmp_path / f"{w}.hip"
        f.write_text(f"int {w}_kernel() {{ return 1; }}\n")
        srcs[w] = [str(f)]
    monkeypatch.setattr(bench, "KERNEL_SRCS", srcs)
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path))
    for w, nbytes in (("wide_head", 300.0), ("hymo", 190.0)):
        (tmp_path / f"traffic_{w}.json").write_text(
            json.dumps({"kernel_sha256_16": bench.kernel_source_hash(w), "bytes_per_launch": nbytes}))
    assert bench.measured_traffic("wide_head") == 300.0
    assert bench.measured_traffic("hymo") == 190.0
    assert bench.measured_traffic("varlen") is None
    (tmp_path / "hymo.hip").write_text("int hymo_kernel() { return 2; }\n")  # the code changed
    assert bench.measured_traffic("hymo") is None
    assert bench.measured_traffic("wide_head") == 300.0


def test_full_width_forward_flops():
    """The training-step line adds the full-width forward: per chunk and
    head 3 C d^2 dense products, four triangular C^2 d ones at half, and one
    triangular inverse (C^3 / 6)."""
    wl = synth.WORKLOADS["wide_head"]
    C, d = 64, 128
    per = 3 * C * d * d + 2 * C * C * d + C ** 3 // 6
    assert bench.fwd_flops_full(wl, [wl.T] * wl.B) == 2 * per * 64 * wl.B * wl.H
    assert bench.fwd_flops_full(wl, [1]) == bench.fwd_flops_full(wl, [64])


def test_train_pass_needs_the_full_width_shapes():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--pass", "train",
                        "--workload", "small_state"], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "dk = dv = 128" in r.stderr
