"""Builds libuq.so (gfx950) in-tree with hipcc.

Usage: python -m bit_kv_cache_wht_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["csrc/uq_api.hip", "csrc/uq_append.hip", "csrc/uq_decode.hip", "csrc/uq_stream.hip"]
LIB = os.path.join(PKG, "libuq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # the write path's rounding decisions must see plain IEEE float64 ops
    "-ffp-contract=off",
    # no packed FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: with the AGPR form the chunked prefill's output
    # accumulators were copied between AGPRs and VGPRs every step (28.1 ms
    # against 30.0 ms on the ragged workload; the decode kernels are unchanged)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(PKG, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
