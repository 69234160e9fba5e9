"""Build libkda.so (HIP kernels + C-ABI runtime) for gfx950 with hipcc.

Run as `python -m kda_chunked_delta_amd.build`; __graft_entry__.build() calls
build() too. The library is written in-tree next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkda.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("kda_kernels.hip", "kda_decode.hip", "kda_runtime.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # deterministic arithmetic: no contraction of separate multiplies and adds,
    # so every kernel that shares a device routine rounds identically
    "-ffp-contract=off",
    # packed fp32 VALU instructions are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
    "-I" + os.path.join(HERE, "csrc"),
]


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the device-only feature flag; drop that note
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
