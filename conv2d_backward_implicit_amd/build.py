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
           os.path.join(CSRC, "forward_gemm.hip"), os.path.join(CSRC, "pointwise_gemm.hip")]
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


def _run(cmd, verbose):
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


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source into LIB_PATH (always recompiles): one object per
    source, compiled in parallel, then linked."""
    from concurrent.futures import ThreadPoolExecutor

    obj_dir = os.path.join(ROOT, "_build", "obj%d" % os.getpid())
    os.makedirs(obj_dir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-shared"] + list(extra_flags)
    objs = [os.path.join(obj_dir, os.path.basename(src) + ".o") for src in SOURCES]
    jobs = max(1, min(len(SOURCES), len(os.sched_getaffinity(0)), 8))
    with ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_run, [hipcc()] + flags + ["-I", INCLUDE, "-I", CSRC, "-c", src,
                                                     "-o", obj], verbose)
                for src, obj in zip(SOURCES, objs)]
        for f in futs:
            f.result()
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    for obj in objs:
        os.remove(obj)
    os.rmdir(obj_dir)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
