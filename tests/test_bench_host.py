"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the algorithmic
byte and flop counts the roofline divides by, and the source hash that
decides whether committed counter readings still describe the kernel."""
import os
import subprocess
import sys

import bench
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


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    h1 = bench.kernel_source_hash()
    src.write_text("/* a note */\nint f(int x)   {\n\n  return x + 1;  // changed comment\n}\n")
    assert bench.kernel_source_hash() == h1
    src.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_source_hash() != h1
