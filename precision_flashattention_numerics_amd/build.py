"""Build the HIP library libpasa_attn.so for gfx950 (in-tree).

hipcc cross-compiles without a GPU.  All device code is built with packed
fp32 arithmetic disabled (the compiler still emits packed fp16 math).
"""
import glob
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpasa_attn.so")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]

# Per-source compiler options (each prefill head dim is its own unit),
# measured A/B in one process with bitwise-equal outputs:
#   * head_dim 64: the compiler's iterative minimum-register scheduling, 4-5 %
#     faster on every head_dim-64 shape tried (the SVD-shaped prefill 312.5
#     against 327.5 us);
#   * head_dim 128 keeps the default: iterative ILP scheduling was 0.7-1.7 %
#     faster on the Qwen2-shaped prefill but 0.6-2.1 % slower on the
#     long-context one (and spilled registers in the naive key-split kernel);
#     minimum-register was 0.5 % slower on the Qwen2 shape.  With the matrix
#     phase laid out by hand both measured within 1.3 % of the default on five
#     shapes;
#   * the decode keeps the default (0.7 % slower with iterative ILP, 11 %
#     slower with minimum-register).
SOURCE_FLAGS = {
    "pasa_fwd_d64.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-minreg"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


PEAK_SRC = os.path.join(HERE, "peak", "peak_probe.hip")
PEAK_LIB = os.path.join(HERE, "peak", "libpasa_peak.so")


def _hipcc(out, srcs, extra, verbose):
    """Compile each source to an object with its own options, then link."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory(prefix="pasa_build_") as d:
        objs = []
        for src in srcs:
            obj = os.path.join(d, os.path.basename(src) + ".o")
            cmd = [hipcc, *FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), *(extra or []),
                   "-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            objs.append(obj)
        cmd = [hipcc, *FLAGS, "-shared", "-o", tmp, *objs]
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
