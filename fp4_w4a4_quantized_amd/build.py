"""Build libfp4q.so (all HIP kernels and the C ABI) for gfx950 with hipcc.

The library is built in place, next to this file, so that it travels with
the source tree; nothing is installed.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp4q.so")
SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "gemm_big.hip", "gemm_skinny.hip", "decompose.hip", "select.hip", "permute.hip", "noalloc.hip"]
# the peak microbenchmarks (measurement only) go into a library of their own
PEAKS_LIB = os.path.join(HERE, "libfp4q_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfp4q)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # every FP32 step of the quantizer is one rounded IEEE operation: no
        # contraction into FMA; correctly rounded division is HIP's default
        "-ffp-contract=off",
        # keep the compiler from forming packed FP32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def _link(out: str, sources: list[str], verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *flags(), "-o", tmp, *[os.path.join(CSRC, s) for s in sources]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose and res.stderr:
        print(res.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every kernel source into libfp4q.so (and the peak
    microbenchmarks into libfp4q_peaks.so); returns libfp4q.so's path."""
    _link(PEAKS_LIB, PEAKS_SOURCES, verbose)
    return _link(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
