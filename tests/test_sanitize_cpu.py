"""CPU sanitizer leg: the oracle and the C ABI's host-side argument validation,
built with the host compiler's address and undefined-behaviour sanitizers.

* The oracle (oracle/oracle.c) is rebuilt with -fsanitize=address,undefined
  and the oracle's pins (tests/test_oracle.py) run against that build in a
  child process; any out-of-bounds access, use after free or undefined
  behaviour in the oracle fails the run.
* The validators every entry point calls before enqueueing work
  (csrc/pasa_validate.hpp, plain host C++) are compiled into
  tests/abi_validate_check.cpp and driven with edge-case sizes.

Neither involves the GPU or the HIP compiler's device code."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

HAVE_GCC = shutil.which("gcc") is not None and shutil.which("g++") is not None
pytestmark = pytest.mark.skipif(not HAVE_GCC, reason="gcc/g++ not available")

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_validation_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_validate_check"
    r = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
         "-o", str(exe), os.path.join(ROOT, "tests", "abi_validate_check.cpp")],
        capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env={**os.environ, **SAN_ENV})
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="no shared ASan runtime")
def test_oracle_pins_under_sanitizers(tmp_path):
    from oracle.build import build
    lib = build(sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    code = ("import sys, pytest\n"
            "import oracle.oracle as o\n"
            f"assert o._LIB_PATH == {lib!r}, o._LIB_PATH\n"
            "rc = pytest.main(['-x', '-q', '-p', 'no:cacheprovider', 'tests/test_oracle.py'])\n"
            "assert o._lib is not None\n"
            "sys.exit(int(rc))\n")
    pre = os.environ.get("LD_PRELOAD")
    env = {**os.environ, **SAN_ENV, "PASA_ORACLE_LIB": lib,
           # the ASan runtime must be loaded before anything it instruments
           "LD_PRELOAD": _runtime("libasan.so") + (":" + pre if pre else "")}
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=900, env=env)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
