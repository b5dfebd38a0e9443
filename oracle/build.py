"""Build the CPU oracle library (test infrastructure only).

Compiles ``oracle.c`` with gcc into ``liboracle.so`` next to this file.  The
oracle shares no source, header or build step with the HIP library.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"]


def build(verbose: bool = False, sanitize: bool = False, out: str = None) -> str:
    """Build liboracle.so; with sanitize=True an address- and
    undefined-behaviour-sanitized copy (to `out`) for the CPU sanitizer test."""
    src = os.path.join(HERE, "oracle.c")
    lib = out or LIB
    tmp = lib + ".tmp"
    opt = SANITIZE_FLAGS if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
