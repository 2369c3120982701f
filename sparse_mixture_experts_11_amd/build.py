"""Build the HIP shared library libmoe.so for gfx950 (in-tree).

Each source compiles to its own object (in parallel) under _build/, then one
link step makes the library.  build() recompiles every source each time it
is called; build(incremental=True) recompiles only sources older than
themselves or any header.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
SO = os.path.join(HERE, "libmoe.so")
SOURCES = ["moe_api.hip", "route.hip", "dispatch.hip", "gemm.hip", "decode.hip", "simt.hip",
           "combine.hip", "qb.hip", "route_bwd.hip", "experts_bwd.hip", "latent_bwd.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # Packed-fp32 VALU forms stay out of generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _headers():
    return glob.glob(os.path.join(CSRC, "*.hpp")) + [os.path.join(ROOT, "include", "moe.h")]


def build(verbose: bool = False, incremental: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ, exist_ok=True)
    newest_header = max(os.path.getmtime(h) for h in _headers())

    def compile_one(src):
        path = os.path.join(CSRC, src)
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        if incremental and os.path.exists(obj) and os.path.getmtime(obj) > max(
                os.path.getmtime(path), newest_header):
            return obj, None
        cmd = [hipcc, *HIPCC_FLAGS, "-c", "-o", obj + ".tmp", path]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            return obj, r.stdout + r.stderr
        os.replace(obj + ".tmp", obj)
        return obj, None

    jobs = int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as pool:
        results = list(pool.map(compile_one, SOURCES))
    errors = [msg for _, msg in results if msg]
    if errors:
        sys.stderr.write("\n".join(errors))
        raise RuntimeError("hipcc failed")
    tmp = SO + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv))
