"""bench.py's command-line contract on the CPU: more than one GPU is refused with a
message (exit status 2) before any GPU work, and the JSON helpers stay importable."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2, r.stdout + r.stderr
    assert "one GPU only" in r.stdout + r.stderr
    assert r.stdout.strip() == "" or not r.stdout.strip().startswith("{")  # no JSON line for a refused run


def test_kernel_source_sha_is_stable():
    sys.path.insert(0, ROOT)
    import bench

    a, b = bench.kernel_source_sha(), bench.kernel_source_sha()
    assert a == b and len(a) == 16
