"""Build the HIP shared library libmoe.so for gfx950 (in-tree)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libmoe.so")
SOURCES = ["moe_api.hip", "route.hip", "dispatch.hip", "gemm.hip", "decode.hip", "simt.hip",
           "combine.hip", "qb.hip", "route_bwd.hip", "experts_bwd.hip", "latent_bwd.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Packed-fp32 VALU forms stay out of generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = SO + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed")
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
