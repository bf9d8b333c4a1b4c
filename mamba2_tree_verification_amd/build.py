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
# HBM ceiling probes for the measurement harness (not part of the ABI)
PROBE_LIB = os.path.join(HERE, "libssm_tree_probe.so")
PROBE_SOURCES = ["probe.hip"]
SOURCES = ["api.hip", "verify.hip", "verify_tt.hip", "verify_fifo.hip", "commit.hip", "commit_verify.hip",
           "plan.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form", "-Wno-unused-command-line-argument"]


def command(out: str, extra=()) -> list:
    """One hipcc line building the whole library (for reference; build()
    compiles the translation units in parallel and links them)."""
    return [hipcc(), *FLAGS, "-shared", *extra, "-o", out, *[os.path.join(CSRC, s) for s in SOURCES]]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libssm_tree.so")


def build(verbose: bool = False, extra=(), jobs: int = 0) -> str:
    """Compile every source of both libraries to object files (in
    parallel), then link each shared library in place, replacing it
    atomically.  Returns the path of libssm_tree.so."""
    from concurrent.futures import ThreadPoolExecutor
    tag = "%d" % os.getpid()
    libs = [(LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)]
    objs = {lib: [os.path.join(CSRC, os.path.splitext(s)[0] + ".o" + tag) for s in srcs] for lib, srcs in libs}
    cmds = [[hipcc(), *FLAGS, *extra, "-c", "-o", o, os.path.join(CSRC, s)]
            for lib, srcs in libs for s, o in zip(srcs, objs[lib])]
    jobs = jobs or min(len(cmds), max(1, min(os.cpu_count() or 1, 16)))
    try:
        with ThreadPoolExecutor(jobs) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        for lib, _ in libs:
            tmp = lib + ".tmp" + tag
            _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs[lib]], verbose)
            os.replace(tmp, lib)
    finally:
        for lib, _ in libs:
            for o in objs[lib]:
                if os.path.exists(o):
                    os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
