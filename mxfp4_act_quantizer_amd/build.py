"""Build libkroquant.so in-tree with hipcc for gfx950.

    python -m mxfp4_act_quantizer_amd.build            # build
    python -m mxfp4_act_quantizer_amd.build --resources  # also print VGPR/LDS use per kernel
"""
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkroquant.so")
SOURCES = ["kq_kernels.hip", "kq_capi.hip", "kq_host.cpp", "kq_measure.hip", "kq_gemm.hip", "kq_adaln.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def source_hash():
    """sha256 (first 16 hex digits) of every source the library is built from:
    csrc/* and include/*, in name order.  Compiled into kq_build_info(), so a
    loaded library can be checked against the tree it should come from."""
    h = hashlib.sha256()
    for d in (CSRC, os.path.join(ROOT, "include")):
        for f in sorted(os.listdir(d)):
            if f.endswith((".hip", ".h", ".cpp")):
                h.update(f.encode())
                with open(os.path.join(d, f), "rb") as fh:
                    h.update(fh.read())
    return h.hexdigest()[:16]


def build(resources=False, verbose=False):
    srcs = [os.path.join(CSRC, f) for f in SOURCES]
    cmd = [HIPCC, *FLAGS, f'-DKQ_SOURCE_HASH="{source_hash()}"', "-o", LIB + ".tmp", *srcs]
    if resources:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "not a recognized feature for this target"
    err = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    os.replace(LIB + ".tmp", LIB)
    if verbose or resources:
        print(err)
    return LIB


if __name__ == "__main__":
    build(resources="--resources" in sys.argv, verbose=True)
    print("built", LIB)
