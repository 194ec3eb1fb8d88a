"""Builds librglru.so in-tree with hipcc for gfx950 (cross-compiles without a GPU)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "librglru.so")
SOURCES = ["rglru_api.cpp", "rglru_gates.hip", "rglru_scan.hip", "rglru_decode.hip",
           "rglru_fused.hip", "rglru_backward.hip", "rglru_bwd_tiles.hip", "rglru_bwd_fused.hip",
           "rglru_mqa.hip", "rglru_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # no packed fp32 (v_pk_*_f32) in generated device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep single-lane atomics (work tickets) as plain atomics: the wave-aggregating rewrite
    # consumes the returned value right after the atomic, which would stall on its round trip
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out, flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
