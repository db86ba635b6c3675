"""Build the HIP library ``libmaxsim_amd.so`` for gfx950 with hipcc.

One shared object holds every kernel and the C ABI of include/maxsim.h. The
library is built in-tree (next to this file) so it travels with the source.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmaxsim_amd.so")
SOURCES = ["abi.hip", "fwd_dense.hip", "fwd_varlen.hip", "fwd_dim.hip", "bwd.hip", "topk.hip", "chamfer.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops stay off in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # device code: scores are finite or -inf, never NaN; with NaNs not honoured
    # and IEEE mode off, a float max is a single v_max_f32/v_max3_f32 with no
    # canonicalisation of its operands
    "-Xarch_device", "-fno-honor-nans", "-Xarch_device", "-mno-amdgpu-ieee",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    """Compile every kernel source into LIB; always recompiles."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
