"""Compile the HIP library in-tree for gfx950: long_document_sparse_amd/liblwattn.so."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "lwattn.hip")
DEPS = [SRC, os.path.join(PKG, "csrc", "kernels.hpp"), os.path.join(PKG, "csrc", "backward.hpp"),
        os.path.join(PKG, "csrc", "causal.hpp"),
        os.path.join(PKG, "csrc", "blocksparse.hpp"),
        os.path.join(PKG, "csrc", "layer.hpp"),
        os.path.join(PKG, "csrc", "probe.hpp"),
        os.path.join(ROOT, "include", "lwattn.h")]
LIB = os.path.join(PKG, "liblwattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs: without it the backward kernels
    # copy their accumulators between AGPRs and VGPRs on every tile
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-inline-asm",
]


def build(verbose: bool = False, extra=None) -> str:
    tmp = LIB + ".tmp"
    # rocBLAS runs the encoder layer's plain GEMMs
    cmd = [HIPCC, *FLAGS, *(extra or []), "-I", os.path.join(ROOT, "include"), "-o", tmp, SRC, "-lrocblas", "-lhipblaslt"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose=True))
