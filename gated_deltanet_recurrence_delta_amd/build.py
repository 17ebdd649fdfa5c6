"""Build the HIP library ``libgdn.so`` for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("gdn_fwd.hip", "gdn_fwd_full.hip", "gdn_recurrent.hip",
                                                "gdn_diag.hip", "gdn_bwd.hip", "gdn_bwd_full.hip")]
LIB = os.path.join(HERE, "libgdn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed-fp32 VALU forms stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results stay in VGPRs: the state, Gram and output products are
    # all post-processed on the VALU, and accumulators in AGPRs would cost a
    # copy per element each way
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # no implicit multiply-add fusion: code that is inlined in more than one
    # place (prologue and loop, unrolled loop halves) must round identically
    # for results to be bitwise reproducible across chunk positions; the
    # kernels spell out every fused multiply-add they want
    "-ffp-contract=off",
    "-I", os.path.join(ROOT, "include"),
]


# Host-side instrumentation only (AddressSanitizer and UBSan on the C entry
# points' argument checks and launch set-up); the device code is unchanged.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    """Compile the csrc/*.hip sources into libgdn.so, or ``out`` (always
    recompiles); ``sanitize`` adds host-side AddressSanitizer/UBSan."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(HOST_SANITIZE if sanitize else []), *SRCS, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
