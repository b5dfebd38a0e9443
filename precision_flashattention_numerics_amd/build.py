"""Build the HIP library libpasa_attn.so for gfx950 (in-tree).

hipcc cross-compiles without a GPU.  All device code is built with packed
fp32 arithmetic disabled (the compiler still emits packed fp16 math).
"""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpasa_attn.so")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


PEAK_SRC = os.path.join(HERE, "peak", "peak_probe.hip")
PEAK_LIB = os.path.join(HERE, "peak", "libpasa_peak.so")


def _hipcc(out, srcs, extra, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS, *(extra or []), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False, extra=None) -> str:
    """The attention library, then the peak microbenchmarks the bench reports
    its roofline fractions against (a separate library, not part of the ABI)."""
    _hipcc(LIB, sources(), extra, verbose)
    _hipcc(PEAK_LIB, [PEAK_SRC], None, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
