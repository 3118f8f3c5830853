"""Build libconv2d_bwd.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m conv2d_backward_implicit_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libconv2d_bwd.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "index_check.hip"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "grad_weight.hip"),
           os.path.join(CSRC, "rms_matmul.hip"), os.path.join(CSRC, "mha_grad_v.hip"),
           os.path.join(CSRC, "forward_gemm.hip")]
ARCH = "gfx950"

# Packed fp32 VALU ops are disabled on purpose: the compiler would otherwise
# form them from ordinary float code.
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source into LIB_PATH (always recompiles)."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra_flags) + ["-I", INCLUDE, "-I", CSRC] \
        + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop
    # only those lines
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
