"""Host-side behaviour that needs no GPU: the binding refuses to run without
its HIP library (there is no fallback path), and the benchmark refuses a
multi-GPU request."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_binding_fails_loudly_without_library(tmp_path):
    pkg = os.path.join(ROOT, "precision_flashattention_numerics_amd")
    dst = tmp_path / "precision_flashattention_numerics_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "csrc", "__pycache__"))
    code = ("import precision_flashattention_numerics_amd as p\n"
            "try:\n    p.attn_fwd\nexcept ImportError as e:\n    print('IMPORT-ERROR', e)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True,
                       timeout=300)
    assert "IMPORT-ERROR" in r.stdout, r.stdout + r.stderr
    assert "libpasa_attn.so" in r.stdout


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_bench_traffic_guard_tracks_sources():
    sys.path.insert(0, ROOT)
    import bench
    h = bench.source_hash()
    assert len(h) == 64
    p, d = bench.recorded_traffic("qwen2")
    f = bench.traffic_file("qwen2")
    text = open(f).read() if os.path.exists(f) else ""
    if f"source_sha256={h}" in text:
        assert p is not None and d is not None
    else:
        assert p is None and d is None


def test_profile_commands_run_committed_files_only():
    """Every rocprofv3 command a profile summary records runs bench.py, which
    is committed, and never a working file."""
    sys.path.insert(0, ROOT)
    import bench
    for set_name in bench.PROFILE_SETS:
        for kind in ("trace", "pmc1", "pmc2", "fetch", "write", "cfetch", "cwrite"):
            cmd = bench.profile_cmd(set_name, kind)
            assert cmd.startswith("rocprofv3 ") and "-- python bench.py" in cmd
            assert "_work" not in cmd
