"""Host-side hardening: the C ABI's argument checks and the C oracle run under
AddressSanitizer and UBSan.

Two instrumented builds go to ``_build/sanitize`` (rebuilt when their sources
change): the HIP library with host-only instrumentation (device code as
usual) and the C oracle.  The ABI tests and the oracle's pins then run in
child processes against them, with the matching sanitizer runtime preloaded;
any sanitizer report fails the test.  Nothing here touches a GPU: the ABI
tests only exercise argument validation, which returns before any launch.
"""
import glob
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
PKG = os.path.join(ROOT, "gated_deltanet_recurrence_delta_amd")
REPORT_MARKERS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _digest(paths):
    h = hashlib.sha256()
    for p in sorted(paths):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _cached(target, sources, make):
    stamp = target + ".src"
    d = _digest(sources)
    if not (os.path.exists(target) and os.path.exists(stamp) and open(stamp).read() == d):
        make(target)
        with open(stamp, "w") as f:
            f.write(d)
    return target


def _run(args, env_extra):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *args],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    text = r.stdout + r.stderr
    return r.returncode, text


def test_oracle_pins_under_asan_ubsan():
    import oracle

    os.makedirs(OUT, exist_ok=True)
    src = os.path.join(ROOT, "oracle", "gdn_oracle.c")
    lib = _cached(os.path.join(OUT, "libgdn_oracle_san.so"), [src],
                  lambda t: oracle.build(force=True, out=t, sanitize=True))
    pre = ":".join(subprocess.check_output(["gcc", f"-print-file-name={n}"], text=True).strip()
                   for n in ("libasan.so", "libubsan.so"))
    rc, text = _run(["tests/test_oracle.py", "tests/test_oracle_mutants.py", "tests/test_oracle_scan.py"],
                    {"GDN_ORACLE_LIB": lib, "LD_PRELOAD": pre})
    assert not any(m in text for m in REPORT_MARKERS), text[-4000:]
    assert rc == 0, text[-4000:]


def test_abi_checks_under_asan_ubsan():
    from gated_deltanet_recurrence_delta_amd import build as hip_build

    rt = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt or not os.path.exists(hip_build.HIPCC):
        pytest.skip("no hipcc / clang sanitizer runtime in this image")
    os.makedirs(OUT, exist_ok=True)
    sources = hip_build.SRCS + glob.glob(os.path.join(PKG, "csrc", "*.h")) + \
        [os.path.join(ROOT, "include", "gdn.h")]
    lib = _cached(os.path.join(OUT, "libgdn_san.so"), sources,
                  lambda t: hip_build.build(out=t, sanitize=True))
    rc, text = _run(["tests/test_abi.py", "-k", "not python_wrapper"],
                    {"GDN_LIB_PATH": lib, "LD_PRELOAD": rt[0]})
    assert not any(m in text for m in REPORT_MARKERS), text[-4000:]
    assert rc == 0, text[-4000:]
