"""Build libssm_tree.so in place with hipcc for gfx950.

Packed-FP32 VALU instructions are disabled for every device translation
unit (``-target-feature -packed-fp32-ops``): the kernels are written with
scalar float arithmetic only.  Matrix-core results are allocated in
ordinary VGPRs (``-amdgpu-mfma-vgpr-form``) rather than AccVGPRs, which
keeps the streaming verify kernel at four waves per SIMD.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssm_tree.so")
SOURCES = ["api.hip", "verify.hip", "verify_mfma.hip", "verify_tt.hip", "verify_fifo.hip", "commit.hip", "commit_verify.hip",
           "plan.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def command(out: str, extra=()) -> list:
    return [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wno-unused-command-line-argument", *extra, "-o", out,
            *[os.path.join(CSRC, s) for s in SOURCES]]


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libssm_tree.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
