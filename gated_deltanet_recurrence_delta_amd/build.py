"""Build the HIP library ``libgdn.so`` for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("gdn_fwd.hip", "gdn_fwd_full.hip", "gdn_recurrent.hip",
                                                "gdn_diag.hip", "gdn_bwd.hip")]
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


def build(verbose: bool = False) -> str:
    """Compile the csrc/*.hip sources into libgdn.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *SRCS, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
