"""Build libmxq.so (the HIP kernels and their C ABI) in-tree for gfx950."""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = ["csrc/quant.hip", "csrc/gemm.hip", "csrc/api.hip"]
LIB = os.path.join(PKG, "libmxq.so")


def source_digest():
    """SHA-256 of the kernel sources and the C header (identifies a build)."""
    import hashlib
    h = hashlib.sha256()
    for rel in SOURCES + ["csrc/common.h"]:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, "include", "mxq.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose=False):
    """Compile every source for gfx950 into block_quant_gemm_amd/libmxq.so."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
           "-I" + os.path.join(ROOT, "include"),
           # keep FP32 arithmetic off the packed-FP32 instructions
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", tmp] + [os.path.join(PKG, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stderr or "").splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
