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


def test_clock_reader_is_absent_without_a_gpu():
    """The in-process metrics reader gives up quietly where no GPU (or no amdsmi) is
    usable, and the clock window then reports nothing rather than failing."""
    sys.path.insert(0, ROOT)
    import bench
    import torch

    if torch.cuda.is_available():
        import pytest

        pytest.skip("a GPU is visible")
    assert bench.smi_reader() is None
    calls = []
    assert bench.sample_clock_under_load(lambda: calls.append(1), 0.1) == ([], [], None)
    assert calls == []  # no launches when there is nothing to read
